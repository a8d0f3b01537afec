/* Oracle projection and SH colour, fp64. TEST INFRASTRUCTURE ONLY.
 *
 * [LOAD-IMB] section 2.1, Eq. 1: each Gaussian has a centre, a covariance
 * built from scale and rotation, an opacity and a colour; the 2D covariance is
 * Sigma' = J W Sigma W^T J^T for the viewing transform W and the Jacobian J of
 * the projection. [3DGS-CUDA] Step 3: the view-dependent colour is the sum over
 * 16 SH basis functions Y_k(d) of Y_k(d) s_k per channel; Step 1 (b): a splat
 * can reach the 1/255 alpha cutoff only where q(d) <= 2 ln(255 o).
 *
 * Readings where the pages are silent: a low-pass variance added to Sigma'
 * (camera argument), pixel centres at +0.5, conic b the off-diagonal entry of
 * Sigma'^-1, real SH without Condon-Shortley phase and no colour offset/clamp,
 * cull when t_z <= znear or tau <= 0.
 */
#include <math.h>
#include <string.h>
#include "oracle.h"

static const double OR_PI = 3.14159265358979323846;

static double fact(int k) {
  double f = 1.0;
  for (int i = 2; i <= k; i++) f *= i;
  return f;
}

/* Associated Legendre functions P_l^m(x), 0 <= m <= l <= 3, without the
   Condon-Shortley phase, by the textbook recurrences. */
static void legendre(double x, double P[4][4]) {
  double s = sqrt(fmax(0.0, 1.0 - x * x));
  memset(P, 0, sizeof(double) * 16);
  P[0][0] = 1.0;
  for (int m = 1; m <= 3; m++) P[m][m] = (2 * m - 1) * s * P[m - 1][m - 1];
  for (int m = 0; m <= 2; m++) P[m + 1][m] = x * (2 * m + 1) * P[m][m];
  for (int l = 2; l <= 3; l++)
    for (int m = 0; m <= l - 2; m++)
      P[l][m] = ((2 * l - 1) * x * P[l - 1][m] - (l + m - 1) * P[l - 2][m]) / (l - m);
}

void or_sh_basis(int degree, const double *d, double *Y) {
  double P[4][4];
  double ct = fmin(1.0, fmax(-1.0, d[2]));
  double phi = atan2(d[1], d[0]);
  legendre(ct, P);
  for (int l = 0; l <= degree; l++) {
    for (int m = -l; m <= l; m++) {
      int am = m < 0 ? -m : m;
      double N = sqrt((2 * l + 1) / (4.0 * OR_PI) * fact(l - am) / fact(l + am));
      double v;
      if (m > 0) v = sqrt(2.0) * N * P[l][am] * cos(am * phi);
      else if (m < 0) v = sqrt(2.0) * N * P[l][am] * sin(am * phi);
      else v = N * P[l][0];
      Y[l * (l + 1) + m] = v;
    }
  }
}

static void project_one(const float *mu_f, const float *ls, const float *qt, float op,
                        const float *sh, int degree, const or_camera *cam, double out[12]) {
  const double *M = cam->w2c;
  double R[3][3] = {{M[0], M[1], M[2]}, {M[4], M[5], M[6]}, {M[8], M[9], M[10]}};
  double tc[3] = {M[3], M[7], M[11]};
  double mu[3] = {mu_f[0], mu_f[1], mu_f[2]};
  memset(out, 0, sizeof(double) * 12);
  out[9] = -1.0;

  /* camera-space centre t = R mu + t_cam */
  double t[3];
  for (int i = 0; i < 3; i++) t[i] = R[i][0] * mu[0] + R[i][1] * mu[1] + R[i][2] * mu[2] + tc[i];
  if (!(t[2] > cam->znear)) return;

  /* unit quaternion (w, x, y, z) -> rotation matrix */
  double w = qt[0], x = qt[1], y = qt[2], z = qt[3];
  double qn = sqrt(w * w + x * x + y * y + z * z);
  if (!(qn > 0)) return;
  w /= qn; x /= qn; y /= qn; z /= qn;
  double Rq[3][3] = {
      {1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)},
      {2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)},
      {2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)}};

  /* Sigma = Rq diag(exp(2 s)) Rq^T */
  double s2[3] = {exp(2.0 * ls[0]), exp(2.0 * ls[1]), exp(2.0 * ls[2])};
  double Sig[3][3];
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double acc = 0;
      for (int k = 0; k < 3; k++) acc += Rq[i][k] * s2[k] * Rq[j][k];
      Sig[i][j] = acc;
    }

  /* camera-space covariance V = R Sigma R^T */
  double RS[3][3], V[3][3];
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double acc = 0;
      for (int k = 0; k < 3; k++) acc += R[i][k] * Sig[k][j];
      RS[i][j] = acc;
    }
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double acc = 0;
      for (int k = 0; k < 3; k++) acc += RS[i][k] * R[j][k];
      V[i][j] = acc;
    }

  /* Jacobian of (fx X/Z + cx, fy Y/Z + cy) at t */
  double iz = 1.0 / t[2];
  double J[2][3] = {{cam->fx * iz, 0.0, -cam->fx * t[0] * iz * iz},
                    {0.0, cam->fy * iz, -cam->fy * t[1] * iz * iz}};
  double JV[2][3], S2[2][2];
  for (int i = 0; i < 2; i++)
    for (int j = 0; j < 3; j++) {
      double acc = 0;
      for (int k = 0; k < 3; k++) acc += J[i][k] * V[k][j];
      JV[i][j] = acc;
    }
  for (int i = 0; i < 2; i++)
    for (int j = 0; j < 2; j++) {
      double acc = 0;
      for (int k = 0; k < 3; k++) acc += JV[i][k] * J[j][k];
      S2[i][j] = acc;
    }
  S2[0][0] += cam->lowpass;
  S2[1][1] += cam->lowpass;
  double sxy = 0.5 * (S2[0][1] + S2[1][0]);
  double det = S2[0][0] * S2[1][1] - sxy * sxy;
  if (!(det > 0)) return;

  double tau = 2.0 * log(255.0 * (double)op);
  if (!((float)tau > 0.0f)) return;

  /* view-dependent colour: direction from the camera centre o = -R^T t_cam */
  double oc[3];
  for (int i = 0; i < 3; i++) oc[i] = -(R[0][i] * tc[0] + R[1][i] * tc[1] + R[2][i] * tc[2]);
  double dv[3] = {mu[0] - oc[0], mu[1] - oc[1], mu[2] - oc[2]};
  double dn = sqrt(dv[0] * dv[0] + dv[1] * dv[1] + dv[2] * dv[2]);
  double rgb[3] = {0, 0, 0};
  if (dn > 0) {
    dv[0] /= dn; dv[1] /= dn; dv[2] /= dn;
    double Y[16];
    int K = (degree + 1) * (degree + 1);
    or_sh_basis(degree, dv, Y);
    for (int k = 0; k < K; k++)
      for (int ch = 0; ch < 3; ch++) rgb[ch] += Y[k] * sh[3 * k + ch];
  }

  out[0] = cam->fx * t[0] * iz + cam->cx;
  out[1] = cam->fy * t[1] * iz + cam->cy;
  out[2] = S2[1][1] / det;
  out[3] = -sxy / det;
  out[4] = S2[0][0] / det;
  out[5] = op;
  out[6] = rgb[0];
  out[7] = rgb[1];
  out[8] = rgb[2];
  out[9] = tau;
  out[10] = t[2];
  out[11] = 0.0;
}

void or_project(int n, const float *means, const float *log_scales, const float *quats,
                const float *opac, const float *sh, int degree, const or_camera *cam,
                float *splats, double *splats64) {
  int K = (degree + 1) * (degree + 1);
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; i++) {
    double rec[12];
    project_one(means + 3 * (int64_t)i, log_scales + 3 * (int64_t)i, quats + 4 * (int64_t)i,
                opac[i], sh + (int64_t)i * K * 3, degree, cam, rec);
    for (int j = 0; j < 12; j++) splats[12 * (int64_t)i + j] = (float)rec[j];
    if (splats[12 * (int64_t)i + 9] <= 0.0f) {
      for (int j = 0; j < 12; j++) splats[12 * (int64_t)i + j] = 0.0f;
      splats[12 * (int64_t)i + 9] = -1.0f;
      rec[9] = -1.0;
    }
    if (splats64)
      for (int j = 0; j < 12; j++) splats64[12 * (int64_t)i + j] = rec[j];
  }
}
