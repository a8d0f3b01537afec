// gs_project: EWA projection of 3D Gaussians to screen-space splats plus SH colour.
//
// "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs",
// section 2.1, Eq. 1: Sigma' = J W Sigma W^T J^T. Here Sigma = (Rq S)(Rq S)^T, so
// Sigma' = (J R Rq S)(J R Rq S)^T: one 2x3 product, then two dot products.
// "What the 3DGS Literature Left on the Table", Step 1 (e) and Step 3: SH colour
// only for visible Gaussians, read as 16-byte vectors; colour = sum_k Y_k(d) s_k.
// The bound tau = 2 ln(255 o) (Step 1 (b)) is computed once here; every later
// decision reads the stored value.
//
// One thread per Gaussian; the kernel is bound by HBM bytes (44 B of geometry
// plus 12 (deg+1)^2 B of SH per visible Gaussian in, 48 B out).
#include "gs_common.h"

namespace {

// Real orthonormal SH basis (no Condon-Shortley phase), index l(l+1)+m, as
// polynomials of the unit direction (x, y, z); constants from
// N_lm = sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) times sqrt(2) for m != 0.
__device__ __forceinline__ void sh_eval(int K, float x, float y, float z, float *Y) {
  Y[0] = 0.28209479177387814f;
  if (K <= 1) return;
  Y[1] = 0.4886025119029199f * y;
  Y[2] = 0.4886025119029199f * z;
  Y[3] = 0.4886025119029199f * x;
  if (K <= 4) return;
  const float xx = x * x, yy = y * y, zz = z * z;
  Y[4] = 1.0925484305920792f * (x * y);
  Y[5] = 1.0925484305920792f * (y * z);
  Y[6] = 0.31539156525252005f * (3.0f * zz - 1.0f);
  Y[7] = 1.0925484305920792f * (x * z);
  Y[8] = 0.5462742152960396f * (xx - yy);
  if (K <= 9) return;
  Y[9] = 0.5900435899266435f * y * (3.0f * xx - yy);
  Y[10] = 2.890611442640554f * (x * y * z);
  Y[11] = 0.4570457994644658f * y * (5.0f * zz - 1.0f);
  Y[12] = 0.3731763325901154f * z * (5.0f * zz - 3.0f);
  Y[13] = 0.4570457994644658f * x * (5.0f * zz - 1.0f);
  Y[14] = 1.445305721320277f * z * (xx - yy);
  Y[15] = 0.5900435899266435f * x * (xx - 3.0f * yy);
}

template <int K>
__global__ void __launch_bounds__(256) k_project(int n, const float *__restrict__ means,
                                                 const float *__restrict__ log_scales,
                                                 const float4 *__restrict__ quats,
                                                 const float *__restrict__ opac,
                                                 const float *__restrict__ sh, CamK cam,
                                                 Splat *__restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float m0 = means[3 * i], m1 = means[3 * i + 1], m2 = means[3 * i + 2];
  const float *R = cam.R;
  const float tx = fmaf(R[0], m0, fmaf(R[1], m1, fmaf(R[2], m2, cam.t[0])));
  const float ty = fmaf(R[3], m0, fmaf(R[4], m1, fmaf(R[5], m2, cam.t[1])));
  const float tz = fmaf(R[6], m0, fmaf(R[7], m1, fmaf(R[8], m2, cam.t[2])));
  const float o = opac[i];
  const float tau = 2.0f * logf(255.0f * o);
  float4 q4 = quats[i];
  const float qn2 = q4.x * q4.x + q4.y * q4.y + q4.z * q4.z + q4.w * q4.w;
  Splat s;
  s.p0 = make_float4(0.f, 0.f, 0.f, 0.f);
  s.p1 = make_float4(0.f, 0.f, 0.f, 0.f);
  s.p2 = make_float4(0.f, -1.0f, 0.f, 0.f);
  if (!(tz > cam.znear) || !(tau > 0.0f) || !(qn2 > 0.0f)) {
    out[i] = s;
    return;
  }
  const float qi = 1.0f / sqrtf(qn2);
  const float w = q4.x * qi, x = q4.y * qi, y = q4.z * qi, z = q4.w * qi;
  // rotation of the unit quaternion (w, x, y, z)
  const float r00 = 1.f - 2.f * (y * y + z * z), r01 = 2.f * (x * y - w * z), r02 = 2.f * (x * z + w * y);
  const float r10 = 2.f * (x * y + w * z), r11 = 1.f - 2.f * (x * x + z * z), r12 = 2.f * (y * z - w * x);
  const float r20 = 2.f * (x * z - w * y), r21 = 2.f * (y * z + w * x), r22 = 1.f - 2.f * (x * x + y * y);
  const float s0 = expf(log_scales[3 * i]), s1 = expf(log_scales[3 * i + 1]),
              s2 = expf(log_scales[3 * i + 2]);
  // columns of Rq S
  const float A00 = r00 * s0, A01 = r01 * s1, A02 = r02 * s2;
  const float A10 = r10 * s0, A11 = r11 * s1, A12 = r12 * s2;
  const float A20 = r20 * s0, A21 = r21 * s1, A22 = r22 * s2;
  // M = R (Rq S), camera-space square root of the covariance
  float M[3][3];
#pragma unroll
  for (int r = 0; r < 3; r++) {
    M[r][0] = R[3 * r] * A00 + R[3 * r + 1] * A10 + R[3 * r + 2] * A20;
    M[r][1] = R[3 * r] * A01 + R[3 * r + 1] * A11 + R[3 * r + 2] * A21;
    M[r][2] = R[3 * r] * A02 + R[3 * r + 1] * A12 + R[3 * r + 2] * A22;
  }
  // rows of J M: J = [[fx/z, 0, -fx x/z^2], [0, fy/z, -fy y/z^2]]
  const float iz = 1.0f / tz;
  const float ux = tx * iz, uy = ty * iz;
  const float fxz = cam.fx * iz, fyz = cam.fy * iz;
  float u[3], v[3];
#pragma unroll
  for (int c = 0; c < 3; c++) {
    u[c] = fxz * (M[0][c] - ux * M[2][c]);
    v[c] = fyz * (M[1][c] - uy * M[2][c]);
  }
  const float uu = u[0] * u[0] + u[1] * u[1] + u[2] * u[2];
  const float vv = v[0] * v[0] + v[1] * v[1] + v[2] * v[2];
  const float uv = u[0] * v[0] + u[1] * v[1] + u[2] * v[2];
  const float cx0 = u[1] * v[2] - u[2] * v[1], cx1 = u[2] * v[0] - u[0] * v[2],
              cx2 = u[0] * v[1] - u[1] * v[0];
  const float lp = cam.lowpass;
  const float sxx = uu + lp, syy = vv + lp;
  // det Sigma' = |u x v|^2 + lp (|u|^2 + |v|^2) + lp^2 (Lagrange identity: no cancellation)
  const float det = (cx0 * cx0 + cx1 * cx1 + cx2 * cx2) + lp * (uu + vv) + lp * lp;
  if (!(det > 0.0f)) {
    out[i] = s;
    return;
  }
  const float idet = 1.0f / det;
  // colour from the view direction
  float d0 = m0 - cam.centre[0], d1 = m1 - cam.centre[1], d2 = m2 - cam.centre[2];
  const float dn2 = d0 * d0 + d1 * d1 + d2 * d2;
  float rgb[3] = {0.f, 0.f, 0.f};
  if (dn2 > 0.0f) {
    const float dinv = 1.0f / sqrtf(dn2);
    d0 *= dinv; d1 *= dinv; d2 *= dinv;
    float Y[16];
    sh_eval(K, d0, d1, d2, Y);
    const float *shi = sh + (size_t)i * (K * 3);
    if constexpr ((K * 3) % 4 == 0) {
      const float4 *sh4 = reinterpret_cast<const float4 *>(shi);
      float buf[K * 3];
#pragma unroll
      for (int j = 0; j < K * 3 / 4; j++) {
        const float4 v4 = sh4[j];
        buf[4 * j] = v4.x; buf[4 * j + 1] = v4.y; buf[4 * j + 2] = v4.z; buf[4 * j + 3] = v4.w;
      }
#pragma unroll
      for (int k = 0; k < K; k++) {
        rgb[0] = fmaf(Y[k], buf[3 * k], rgb[0]);
        rgb[1] = fmaf(Y[k], buf[3 * k + 1], rgb[1]);
        rgb[2] = fmaf(Y[k], buf[3 * k + 2], rgb[2]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < K; k++) {
        rgb[0] = fmaf(Y[k], shi[3 * k], rgb[0]);
        rgb[1] = fmaf(Y[k], shi[3 * k + 1], rgb[1]);
        rgb[2] = fmaf(Y[k], shi[3 * k + 2], rgb[2]);
      }
    }
  }
  s.p0 = make_float4(fmaf(cam.fx, ux, cam.cx), fmaf(cam.fy, uy, cam.cy), syy * idet, -uv * idet);
  s.p1 = make_float4(sxx * idet, o, rgb[0], rgb[1]);
  s.p2 = make_float4(rgb[2], tau, tz, 0.0f);
  out[i] = s;
}

}  // namespace

hipError_t gs_launch_project(int n, const float *means, const float *log_scales, const float *quats,
                             const float *opac, const float *sh, int degree, const CamK &cam,
                             float *splats, hipStream_t st) {
  if (n == 0) return hipSuccess;
  dim3 grid(gs_div_up(n, 256)), block(256);
  const float4 *q4 = reinterpret_cast<const float4 *>(quats);
  Splat *out = reinterpret_cast<Splat *>(splats);
  switch (degree) {
    case 0: hipLaunchKernelGGL(k_project<1>, grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, out); break;
    case 1: hipLaunchKernelGGL(k_project<4>, grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, out); break;
    case 2: hipLaunchKernelGGL(k_project<9>, grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, out); break;
    default: hipLaunchKernelGGL(k_project<16>, grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, out); break;
  }
  return hipGetLastError();
}
