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

static void project_one(const double *mu, const double *ls, const double *qt, double op,
                        const double *sh, int degree, const or_camera *cam, double out[12]) {
  const double *M = cam->w2c;
  double R[3][3] = {{M[0], M[1], M[2]}, {M[4], M[5], M[6]}, {M[8], M[9], M[10]}};
  double tc[3] = {M[3], M[7], M[11]};
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

  double tau = 2.0 * log(255.0 * op);
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

/* One Gaussian's fp32 inputs, widened exactly to fp64. */
static void widen(int i, const float *means, const float *log_scales, const float *quats,
                  const float *opac, const float *sh, int K, double mu[3], double ls[3],
                  double qt[4], double *op, double shd[48]) {
  for (int j = 0; j < 3; j++) {
    mu[j] = means[3 * (int64_t)i + j];
    ls[j] = log_scales[3 * (int64_t)i + j];
  }
  for (int j = 0; j < 4; j++) qt[j] = quats[4 * (int64_t)i + j];
  *op = opac[i];
  for (int j = 0; j < 3 * K; j++) shd[j] = sh[(int64_t)i * K * 3 + j];
}

void or_project(int n, const float *means, const float *log_scales, const float *quats,
                const float *opac, const float *sh, int degree, const or_camera *cam,
                float *splats, double *splats64) {
  int K = (degree + 1) * (degree + 1);
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; i++) {
    double rec[12], mu[3], ls[3], qt[4], op, shd[48];
    widen(i, means, log_scales, quats, opac, sh, K, mu, ls, qt, &op, shd);
    project_one(mu, ls, qt, op, shd, degree, cam, rec);
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

/* The same projection on fp64 inputs (records in fp64 only): the reference that
   finite differences of the backward below are taken on. */
void or_project64(int n, const double *means, const double *log_scales, const double *quats,
                  const double *opac, const double *sh, int degree, const or_camera *cam,
                  double *splats64) {
  int K = (degree + 1) * (degree + 1);
  for (int i = 0; i < n; i++)
    project_one(means + 3 * (int64_t)i, log_scales + 3 * (int64_t)i, quats + 4 * (int64_t)i,
                opac[i], sh + (int64_t)i * K * 3, degree, cam, splats64 + 12 * (int64_t)i);
}

/* The basis of or_sh_basis as polynomials of the direction (x, y, z) and their
   gradients in R^3 (only the part tangent to the sphere matters below). The
   constants are the normalisation N_lm (times sqrt 2 for m != 0) written out. */
void or_sh_cart(int degree, const double *d, double *Y, double *dY) {
  const double x = d[0], y = d[1], z = d[2], pi = OR_PI;
  const double c0 = sqrt(1.0 / (4 * pi)), c1 = sqrt(3.0 / (4 * pi));
  const double c2a = sqrt(15.0 / (4 * pi)), c2b = sqrt(5.0 / (16 * pi)), c2c = sqrt(15.0 / (16 * pi));
  const double c3a = sqrt(35.0 / (32 * pi)), c3b = sqrt(105.0 / (4 * pi)), c3c = sqrt(21.0 / (32 * pi));
  const double c3d = sqrt(7.0 / (16 * pi)), c3e = sqrt(105.0 / (16 * pi));
  const double v[16] = {c0,
                        c1 * y, c1 * z, c1 * x,
                        c2a * x * y, c2a * y * z, c2b * (3 * z * z - 1), c2a * x * z, c2c * (x * x - y * y),
                        c3a * y * (3 * x * x - y * y), c3b * x * y * z, c3c * y * (5 * z * z - 1),
                        c3d * z * (5 * z * z - 3), c3c * x * (5 * z * z - 1), c3e * z * (x * x - y * y),
                        c3a * x * (x * x - 3 * y * y)};
  const double g[16][3] = {{0, 0, 0},
                           {0, c1, 0}, {0, 0, c1}, {c1, 0, 0},
                           {c2a * y, c2a * x, 0}, {0, c2a * z, c2a * y}, {0, 0, 6 * c2b * z},
                           {c2a * z, 0, c2a * x}, {2 * c2c * x, -2 * c2c * y, 0},
                           {6 * c3a * x * y, c3a * (3 * x * x - 3 * y * y), 0},
                           {c3b * y * z, c3b * x * z, c3b * x * y},
                           {0, c3c * (5 * z * z - 1), 10 * c3c * y * z},
                           {0, 0, c3d * (15 * z * z - 3)},
                           {c3c * (5 * z * z - 1), 0, 10 * c3c * x * z},
                           {2 * c3e * x * z, -2 * c3e * y * z, c3e * (x * x - y * y)},
                           {c3a * (3 * x * x - 3 * y * y), -6 * c3a * x * y, 0}};
  const int K = (degree + 1) * (degree + 1);
  for (int k = 0; k < K; k++) {
    Y[k] = v[k];
    for (int j = 0; j < 3; j++) dY[3 * k + j] = g[k][j];
  }
}

static void mat3_mul(const double A[3][3], const double B[3][3], double C[3][3]) {
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double acc = 0;
      for (int k = 0; k < 3; k++) acc += A[i][k] * B[k][j];
      C[i][j] = acc;
    }
}

/* Vector-Jacobian product of the projection for one Gaussian: given dL/d of the
   record's first nine entries (mx, my, a, b, c, o, r, g, b), the gradient with
   respect to the mean, the log-scales, the (unnormalised) quaternion, the
   opacity and the SH coefficients. tau (a decision threshold) and depth (the
   sort key) pass no gradient. A culled Gaussian gets zeros. The chain, in the
   order of the forward pass (section 2.1, Eq. 1 of [LOAD-IMB]; the SH term of
   [3DGS-CUDA] Step 3):
     Lambda = Sigma'^-1        dL/dSigma' = -Lambda G Lambda, G the symmetric
                               gradient of Lambda (b sits on both off-diagonals)
     Sigma' = J V J^T + lp I   dL/dV = J^T dL/dSigma' J, dL/dJ = 2 dL/dSigma' J V
     V = R Sigma R^T           dL/dSigma = R^T dL/dV R
     Sigma = Rq D Rq^T         dL/dRq = 2 dL/dSigma Rq D, dL/dD = diag(Rq^T dL/dSigma Rq)
     D = diag(exp(2 s))        dL/ds = 2 D dL/dD
     Rq = R(q / |q|)           through the rotation-matrix entries, then the
                               projection onto the tangent of the unit sphere
     t = R mu + t_cam          J(t) and the centre (fx t_x / t_z + cx, ...)
     colour = sum_k Y_k(d) s_k d = (mu - o_cam) / |mu - o_cam| */
static void project_bwd_one(const double *mu, const double *ls, const double *qt, double op,
                            const double *sh, int degree, const or_camera *cam, const double *gs,
                            double *gmu, double *gls, double *gq, double *gop, double *gsh) {
  const int K = (degree + 1) * (degree + 1);
  for (int j = 0; j < 3; j++) gmu[j] = gls[j] = 0;
  for (int j = 0; j < 4; j++) gq[j] = 0;
  *gop = 0;
  for (int j = 0; j < 3 * K; j++) gsh[j] = 0;
  double rec[12];
  project_one(mu, ls, qt, op, sh, degree, cam, rec);
  if (!(rec[9] > 0)) return; /* culled */

  const double *M = cam->w2c;
  double R[3][3] = {{M[0], M[1], M[2]}, {M[4], M[5], M[6]}, {M[8], M[9], M[10]}};
  double t[3];
  for (int i = 0; i < 3; i++) t[i] = R[i][0] * mu[0] + R[i][1] * mu[1] + R[i][2] * mu[2] + M[4 * i + 3];
  double qn = sqrt(qt[0] * qt[0] + qt[1] * qt[1] + qt[2] * qt[2] + qt[3] * qt[3]);
  double w = qt[0] / qn, x = qt[1] / qn, y = qt[2] / qn, z = qt[3] / qn;
  double Rq[3][3] = {
      {1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)},
      {2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)},
      {2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)}};
  double D[3] = {exp(2 * ls[0]), exp(2 * ls[1]), exp(2 * ls[2])};
  double Sig[3][3], V[3][3], tmp[3][3], Rt[3][3];
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double acc = 0;
      for (int k = 0; k < 3; k++) acc += Rq[i][k] * D[k] * Rq[j][k];
      Sig[i][j] = acc;
      Rt[i][j] = R[j][i];
    }
  mat3_mul(R, Sig, tmp);
  mat3_mul(tmp, Rt, V);
  double iz = 1.0 / t[2];
  double J[2][3] = {{cam->fx * iz, 0.0, -cam->fx * t[0] * iz * iz},
                    {0.0, cam->fy * iz, -cam->fy * t[1] * iz * iz}};
  double S2[2][2] = {{0, 0}, {0, 0}};
  for (int i = 0; i < 2; i++)
    for (int j = 0; j < 2; j++)
      for (int k = 0; k < 3; k++)
        for (int l = 0; l < 3; l++) S2[i][j] += J[i][k] * V[k][l] * J[j][l];
  S2[0][0] += cam->lowpass;
  S2[1][1] += cam->lowpass;
  double sxy = 0.5 * (S2[0][1] + S2[1][0]);
  double det = S2[0][0] * S2[1][1] - sxy * sxy;
  double L[2][2] = {{S2[1][1] / det, -sxy / det}, {-sxy / det, S2[0][0] / det}};

  /* conic -> Sigma' */
  double G[2][2] = {{gs[2], 0.5 * gs[3]}, {0.5 * gs[3], gs[4]}};
  double GS[2][2];
  for (int i = 0; i < 2; i++)
    for (int j = 0; j < 2; j++) {
      double acc = 0;
      for (int k = 0; k < 2; k++)
        for (int l = 0; l < 2; l++) acc += L[i][k] * G[k][l] * L[l][j];
      GS[i][j] = -acc;
    }
  /* Sigma' -> V and J */
  double GV[3][3], GJ[2][3];
  for (int k = 0; k < 3; k++)
    for (int l = 0; l < 3; l++) {
      double acc = 0;
      for (int i = 0; i < 2; i++)
        for (int j = 0; j < 2; j++) acc += J[i][k] * GS[i][j] * J[j][l];
      GV[k][l] = acc;
    }
  for (int i = 0; i < 2; i++)
    for (int k = 0; k < 3; k++) {
      double acc = 0;
      for (int j = 0; j < 2; j++)
        for (int l = 0; l < 3; l++) acc += GS[i][j] * J[j][l] * V[l][k];
      GJ[i][k] = 2 * acc;
    }
  /* V -> Sigma -> (Rq, D) */
  double GSig[3][3];
  mat3_mul(Rt, GV, tmp);
  mat3_mul(tmp, R, GSig);
  double GRq[3][3], GD[3];
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double acc = 0;
      for (int k = 0; k < 3; k++) acc += GSig[i][k] * Rq[k][j];
      GRq[i][j] = 2 * acc * D[j];
    }
  for (int j = 0; j < 3; j++) {
    double acc = 0;
    for (int i = 0; i < 3; i++)
      for (int k = 0; k < 3; k++) acc += Rq[i][j] * GSig[i][k] * Rq[k][j];
    GD[j] = acc;
    gls[j] = 2 * D[j] * GD[j];
  }
  /* rotation-matrix entries -> unit quaternion -> quaternion */
  const double (*g)[3] = GRq;
  double gw = 2 * (-z * g[0][1] + y * g[0][2] + z * g[1][0] - x * g[1][2] - y * g[2][0] + x * g[2][1]);
  double gx = 2 * (y * g[0][1] + z * g[0][2] + y * g[1][0] - 2 * x * g[1][1] - w * g[1][2] +
                   z * g[2][0] + w * g[2][1] - 2 * x * g[2][2]);
  double gy = 2 * (-2 * y * g[0][0] + x * g[0][1] + w * g[0][2] + x * g[1][0] + z * g[1][2] -
                   w * g[2][0] + z * g[2][1] - 2 * y * g[2][2]);
  double gz = 2 * (-2 * z * g[0][0] - w * g[0][1] + x * g[0][2] + w * g[1][0] - 2 * z * g[1][1] +
                   y * g[1][2] + x * g[2][0] + y * g[2][1]);
  double qd = w * gw + x * gx + y * gy + z * gz;
  gq[0] = (gw - w * qd) / qn;
  gq[1] = (gx - x * qd) / qn;
  gq[2] = (gy - y * qd) / qn;
  gq[3] = (gz - z * qd) / qn;
  /* J(t) and the projected centre -> t -> mu */
  double fx = cam->fx, fy = cam->fy;
  double gt[3];
  gt[0] = GJ[0][2] * (-fx * iz * iz) + gs[0] * fx * iz;
  gt[1] = GJ[1][2] * (-fy * iz * iz) + gs[1] * fy * iz;
  gt[2] = GJ[0][0] * (-fx * iz * iz) + GJ[0][2] * (2 * fx * t[0] * iz * iz * iz) +
          GJ[1][1] * (-fy * iz * iz) + GJ[1][2] * (2 * fy * t[1] * iz * iz * iz) -
          gs[0] * fx * t[0] * iz * iz - gs[1] * fy * t[1] * iz * iz;
  for (int j = 0; j < 3; j++) gmu[j] = R[0][j] * gt[0] + R[1][j] * gt[1] + R[2][j] * gt[2];
  /* opacity, colour */
  *gop = gs[5];
  double oc[3];
  for (int i = 0; i < 3; i++) oc[i] = -(R[0][i] * M[3] + R[1][i] * M[7] + R[2][i] * M[11]);
  double dv[3] = {mu[0] - oc[0], mu[1] - oc[1], mu[2] - oc[2]};
  double dn = sqrt(dv[0] * dv[0] + dv[1] * dv[1] + dv[2] * dv[2]);
  if (!(dn > 0)) return;
  for (int j = 0; j < 3; j++) dv[j] /= dn;
  double Y[16], dY[48], Yl[16];
  or_sh_basis(degree, dv, Yl);
  or_sh_cart(degree, dv, Y, dY);
  double gd[3] = {0, 0, 0};
  for (int k = 0; k < K; k++) {
    double sg = 0;
    for (int ch = 0; ch < 3; ch++) {
      gsh[3 * k + ch] = Yl[k] * gs[6 + ch];
      sg += sh[3 * k + ch] * gs[6 + ch];
    }
    for (int j = 0; j < 3; j++) gd[j] += dY[3 * k + j] * sg;
  }
  double dd = gd[0] * dv[0] + gd[1] * dv[1] + gd[2] * dv[2];
  for (int j = 0; j < 3; j++) gmu[j] += (gd[j] - dv[j] * dd) / dn;
}

void or_project_bwd(int n, const float *means, const float *log_scales, const float *quats,
                    const float *opac, const float *sh, int degree, const or_camera *cam,
                    const double *dsplat, double *gmeans, double *gls, double *gquats,
                    double *gopac, double *gsh) {
  int K = (degree + 1) * (degree + 1);
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; i++) {
    double mu[3], ls[3], qt[4], op, shd[48];
    widen(i, means, log_scales, quats, opac, sh, K, mu, ls, qt, &op, shd);
    project_bwd_one(mu, ls, qt, op, shd, degree, cam, dsplat + 9 * (int64_t)i,
                    gmeans + 3 * (int64_t)i, gls + 3 * (int64_t)i, gquats + 4 * (int64_t)i,
                    gopac + i, gsh + (int64_t)i * K * 3);
  }
}
