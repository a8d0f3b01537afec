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

// One Gaussian's K x 3 SH coefficients into fp32 registers. Stored as fp32 (read
// as 16-byte vectors when the row is a multiple of four floats) or as bf16 bits
// (widened exactly: the 16 bits are the high half of the fp32 word; read as 16-
// or 8-byte vectors when the row allows).
template <int K>
__device__ __forceinline__ void load_sh_row(const float *shi, float *buf) {
  if constexpr ((K * 3) % 4 == 0) {
    const float4 *sh4 = reinterpret_cast<const float4 *>(shi);
#pragma unroll
    for (int j = 0; j < K * 3 / 4; j++) {
      const float4 v4 = sh4[j];
      buf[4 * j] = v4.x; buf[4 * j + 1] = v4.y; buf[4 * j + 2] = v4.z; buf[4 * j + 3] = v4.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < K * 3; j++) buf[j] = shi[j];
  }
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

template <int K>
__device__ __forceinline__ void load_sh_row(const uint16_t *shi, float *buf) {
  if constexpr ((K * 3) % 8 == 0) {
    const uint4 *s4 = reinterpret_cast<const uint4 *>(shi);
#pragma unroll
    for (int j = 0; j < K * 3 / 8; j++) {
      const uint4 v = s4[j];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; h++) {
        buf[8 * j + 2 * h] = bf16_to_f32(w[h] & 0xFFFFu);
        buf[8 * j + 2 * h + 1] = bf16_to_f32(w[h] >> 16);
      }
    }
  } else if constexpr ((K * 3) % 4 == 0) {
    const uint2 *s2 = reinterpret_cast<const uint2 *>(shi);
#pragma unroll
    for (int j = 0; j < K * 3 / 4; j++) {
      const uint2 v = s2[j];
      buf[4 * j] = bf16_to_f32(v.x & 0xFFFFu);
      buf[4 * j + 1] = bf16_to_f32(v.x >> 16);
      buf[4 * j + 2] = bf16_to_f32(v.y & 0xFFFFu);
      buf[4 * j + 3] = bf16_to_f32(v.y >> 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < K * 3; j++) buf[j] = bf16_to_f32(shi[j]);
  }
}

// SH rows moved between HBM and registers through LDS, one wave's 64 rows at a
// time: a row of BYTES bytes is V 16-byte vectors (V = 0: the row is not a whole
// number of vectors and is read per lane instead). Lane l moves vectors l,
// l + 64, ... of the wave's contiguous block, so each load or store instruction
// covers 1 KB of consecutive addresses; a lane reading its own row straight
// from HBM would touch a different cache line in each of its 64 lanes and
// fetch every line once per vector it holds. LDS rows are padded to an odd
// number of vectors (SV), so 16 lanes reading 16-byte vectors at the row
// stride hit distinct banks.
template <int BYTES>
struct RowVecs {
  static constexpr int V = BYTES % 16 == 0 ? BYTES / 16 : 0;
  static constexpr int SV = V % 2 ? V : V + 1;
};

// Load rows [w0, w0 + 64) (src points at row w0), row r only where bit r of
// `want` is set, into this wave's LDS rows; each lane then reads its own row.
template <int V, int SV>
__device__ __forceinline__ void stage_rows_in(const uint4 *__restrict__ src, uint64_t want,
                                              uint4 *lds, int lane) {
  uint4 t[V];
#pragma unroll
  for (int j = 0; j < V; j++) {
    const int f = j * 64 + lane, r = f / V;
    t[j] = ((want >> r) & 1) ? src[f] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int j = 0; j < V; j++) {
    const int f = j * 64 + lane, r = f / V;
    lds[r * SV + (f - r * V)] = t[j];
  }
  wave_sync();
}

// Store this wave's LDS rows [0, rows) to dst (row w0) with whole-wave vectors;
// with acc, add them (as floats) to what dst holds.
template <int V, int SV>
__device__ __forceinline__ void stage_rows_out(uint4 *__restrict__ dst, int rows, const uint4 *lds,
                                               int lane, bool acc = false) {
  wave_sync();
#pragma unroll
  for (int j = 0; j < V; j++) {
    const int f = j * 64 + lane, r = f / V;
    if (r < rows) {
      uint4 v = lds[r * SV + (f - r * V)];
      if (acc) {
        const uint4 o = dst[f];
        v = make_uint4(__float_as_uint(__uint_as_float(o.x) + __uint_as_float(v.x)),
                       __float_as_uint(__uint_as_float(o.y) + __uint_as_float(v.y)),
                       __float_as_uint(__uint_as_float(o.z) + __uint_as_float(v.z)),
                       __float_as_uint(__uint_as_float(o.w) + __uint_as_float(v.w)));
      }
      dst[f] = v;
    }
  }
}

// 16-byte vectors of stored SH coefficients to fp32 (bf16: the upper half of
// the fp32 word, exact).
__device__ __forceinline__ void unpack_vec(const uint4 &v, float *out, const float *) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack_vec(const uint4 &v, float *out, const uint16_t *) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int h = 0; h < 4; h++) {
    out[2 * h] = __uint_as_float(w[h] << 16);
    out[2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
  }
}

// This Gaussian's SH row into buf (K * 3 floats) when `need`; every lane of the
// wave calls it (the staged form is wave-cooperative).
template <int K, typename ShT>
__device__ __forceinline__ void read_sh(const ShT *__restrict__ sh, int i, bool need, float *buf,
                                        uint4 *lds_wave) {
  using RV = RowVecs<K * 3 * (int)sizeof(ShT)>;
  if constexpr (RV::V > 0) {
    const int lane = threadIdx.x & 63;
    const int w0 = i - lane;
    const uint64_t want = wave_ballot(need);
    if (want == 0) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(sh) + (size_t)w0 * RV::V;
    stage_rows_in<RV::V, RV::SV>(src, want, lds_wave, lane);
    if (need) {
      constexpr int PER = 16 / (int)sizeof(ShT);
#pragma unroll
      for (int j = 0; j < RV::V; j++)
        unpack_vec(lds_wave[lane * RV::SV + j], buf + PER * j, sh);
    }
  } else {
    if (need) load_sh_row<K>(sh + (size_t)i * (K * 3), buf);
  }
}

template <int K, typename ShT>
__global__ void __launch_bounds__(256) k_project(int n, const float *__restrict__ means,
                                                 const float *__restrict__ log_scales,
                                                 const float4 *__restrict__ quats,
                                                 const float *__restrict__ opac,
                                                 const ShT *__restrict__ sh, CamK cam,
                                                 Splat *__restrict__ out) {
  using RV = RowVecs<K * 3 * (int)sizeof(ShT)>;  // SH rows read
  using RS = RowVecs<(int)sizeof(Splat)>;         // records written
  constexpr int SV = RV::SV > RS::SV ? RV::SV : RS::SV;
  __shared__ uint4 s_rows[4 * 64 * SV];
  uint4 *lds_wave = s_rows + (threadIdx.x >> 6) * 64 * SV;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  Splat s;
  s.p0 = make_float4(0.f, 0.f, 0.f, 0.f);
  s.p1 = make_float4(0.f, 0.f, 0.f, 0.f);
  const float vbits = __int_as_float(cam.view);  // the record's view (pad word)
  s.p2 = make_float4(0.f, -1.0f, 0.f, vbits);
  bool need_sh = false;
  float d0 = 0.f, d1 = 0.f, d2 = 0.f;
  if (i < n) {
    const float m0 = means[3 * i], m1 = means[3 * i + 1], m2 = means[3 * i + 2];
    const float *R = cam.R;
    const float tx = fmaf(R[0], m0, fmaf(R[1], m1, fmaf(R[2], m2, cam.t[0])));
    const float ty = fmaf(R[3], m0, fmaf(R[4], m1, fmaf(R[5], m2, cam.t[1])));
    const float tz = fmaf(R[6], m0, fmaf(R[7], m1, fmaf(R[8], m2, cam.t[2])));
    const float o = opac[i];
    const float tau = 2.0f * logf(255.0f * o);
    float4 q4 = quats[i];
    const float qn2 = q4.x * q4.x + q4.y * q4.y + q4.z * q4.z + q4.w * q4.w;
    if (tz > cam.znear && tau > 0.0f && qn2 > 0.0f) {
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
      if (det > 0.0f) {
        const float idet = 1.0f / det;
        s.p0 = make_float4(fmaf(cam.fx, ux, cam.cx), fmaf(cam.fy, uy, cam.cy), syy * idet,
                           -uv * idet);
        s.p1 = make_float4(sxx * idet, o, 0.f, 0.f);
        s.p2 = make_float4(0.f, tau, tz, vbits);
        // colour from the view direction
        d0 = m0 - cam.centre[0]; d1 = m1 - cam.centre[1]; d2 = m2 - cam.centre[2];
        const float dn2 = d0 * d0 + d1 * d1 + d2 * d2;
        if (dn2 > 0.0f) {
          const float dinv = 1.0f / sqrtf(dn2);
          d0 *= dinv; d1 *= dinv; d2 *= dinv;
          need_sh = true;
        }
      }
    }
  }
  float buf[K * 3];
  read_sh<K>(sh, i, need_sh, buf, lds_wave);
  if (need_sh) {
    float Y[16];
    sh_eval(K, d0, d1, d2, Y);
    float rgb[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; k++) {
      rgb[0] = fmaf(Y[k], buf[3 * k], rgb[0]);
      rgb[1] = fmaf(Y[k], buf[3 * k + 1], rgb[1]);
      rgb[2] = fmaf(Y[k], buf[3 * k + 2], rgb[2]);
    }
    s.p1.z = rgb[0];
    s.p1.w = rgb[1];
    s.p2.x = rgb[2];
  }
  // the wave's 64 records leave as three 1 KB runs
  const int lane = threadIdx.x & 63;
  const int w0 = i - lane;
  if (w0 < n) {
    wave_sync();  // the LDS rows read above are reused
    lds_wave[lane * RS::SV] = make_uint4(__float_as_uint(s.p0.x), __float_as_uint(s.p0.y),
                                         __float_as_uint(s.p0.z), __float_as_uint(s.p0.w));
    lds_wave[lane * RS::SV + 1] = make_uint4(__float_as_uint(s.p1.x), __float_as_uint(s.p1.y),
                                             __float_as_uint(s.p1.z), __float_as_uint(s.p1.w));
    lds_wave[lane * RS::SV + 2] = make_uint4(__float_as_uint(s.p2.x), __float_as_uint(s.p2.y),
                                             __float_as_uint(s.p2.z), __float_as_uint(s.p2.w));
    stage_rows_out<RS::V, RS::SV>(reinterpret_cast<uint4 *>(out) + (size_t)w0 * RS::V,
                                  min(64, n - w0), lds_wave, lane);
  }
}

// Accumulate sum_k grad Y_k(x, y, z) w_k into (g0, g1, g2): the gradients of
// the polynomials of sh_eval in R^3 (the caller keeps the part tangent to the
// sphere).
__device__ __forceinline__ void sh_grad_acc(int K, float x, float y, float z, const float *w,
                                            float &g0, float &g1, float &g2) {
  if (K <= 1) return;
  const float c1 = 0.4886025119029199f;
  g0 = fmaf(c1, w[3], g0);
  g1 = fmaf(c1, w[1], g1);
  g2 = fmaf(c1, w[2], g2);
  if (K <= 4) return;
  const float c2a = 1.0925484305920792f, c2b = 0.31539156525252005f, c2c = 0.5462742152960396f;
  // Y4 = c2a x y, Y5 = c2a y z, Y6 = c2b (3 z^2 - 1), Y7 = c2a x z, Y8 = c2c (x^2 - y^2)
  g0 += c2a * (y * w[4] + z * w[7]) + 2.0f * c2c * x * w[8];
  g1 += c2a * (x * w[4] + z * w[5]) - 2.0f * c2c * y * w[8];
  g2 += c2a * (y * w[5] + x * w[7]) + 6.0f * c2b * z * w[6];
  if (K <= 9) return;
  const float c3a = 0.5900435899266435f, c3b = 2.890611442640554f, c3c = 0.4570457994644658f,
              c3d = 0.3731763325901154f, c3e = 1.445305721320277f;
  const float xx = x * x, yy = y * y, zz = z * z;
  // Y9 = c3a y (3x^2 - y^2), Y10 = c3b x y z, Y11 = c3c y (5z^2 - 1), Y12 = c3d z (5z^2 - 3),
  // Y13 = c3c x (5z^2 - 1), Y14 = c3e z (x^2 - y^2), Y15 = c3a x (x^2 - 3y^2)
  g0 += 6.0f * c3a * x * y * w[9] + c3b * y * z * w[10] + c3c * (5.0f * zz - 1.0f) * w[13] +
        2.0f * c3e * x * z * w[14] + 3.0f * c3a * (xx - yy) * w[15];
  g1 += 3.0f * c3a * (xx - yy) * w[9] + c3b * x * z * w[10] + c3c * (5.0f * zz - 1.0f) * w[11] -
        2.0f * c3e * y * z * w[14] - 6.0f * c3a * x * y * w[15];
  g2 += c3b * x * y * w[10] + 10.0f * c3c * y * z * w[11] + c3d * (15.0f * zz - 3.0f) * w[12] +
        10.0f * c3c * x * z * w[13] + c3e * (xx - yy) * w[14];
}

// Backward of k_project: the 9 screen-space gradients of a splat record (mx, my,
// a, b, c, o, r, g, b) chained to the Gaussian's mean, log-scales, quaternion,
// opacity and SH coefficients ([LOAD-IMB] section 2.1 Eq. 1 differentiated;
// [3DGS-CUDA] Step 3: dL/ds_k = Y_k(d) dL/dc plus the view-direction term).
// The forward's intermediates are recomputed. tau and depth pass no gradient;
// every output row is written (zeros for a culled Gaussian). A Gaussian no
// pixel touched has an all-zero gradient row, hence all-zero outputs: its
// parameters and SH are not read ([3DGS-CUDA] Step 4, touched-gating).
template <int K, typename ShT>
__global__ void __launch_bounds__(256) k_project_bwd(
    int n, const float *__restrict__ means, const float *__restrict__ log_scales,
    const float4 *__restrict__ quats, const float *__restrict__ opac, const ShT *__restrict__ sh,
    CamK cam, const float *__restrict__ dsplat, float *__restrict__ gmeans,
    float *__restrict__ gls, float4 *__restrict__ gquats, float *__restrict__ gopac,
    float *__restrict__ gsh, bool acc) {
  using RI = RowVecs<K * 3 * (int)sizeof(ShT)>;  // SH rows read
  using RO = RowVecs<K * 3 * 4>;                 // SH gradient rows written (fp32)
  constexpr int SV = RI::SV > RO::SV ? RI::SV : RO::SV;
  __shared__ uint4 s_rows[(RI::V > 0 || RO::V > 0) ? 4 * 64 * SV : 1];
  uint4 *lds_wave = s_rows + (threadIdx.x >> 6) * 64 * SV;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  float gsp[9];
  bool touched = false;
  if (i < n) {
#pragma unroll
    for (int j = 0; j < 9; j++) gsp[j] = dsplat[9 * (size_t)i + j];
#pragma unroll
    for (int j = 0; j < 9; j++) touched = touched || gsp[j] != 0.0f;
  }
  // outputs of a culled or untouched Gaussian stay zero
  float g0 = 0.f, g1 = 0.f, g2 = 0.f;
  float4 gq = make_float4(0.f, 0.f, 0.f, 0.f);
  float dls[3] = {0.f, 0.f, 0.f}, gop = 0.f;
  float d0 = 0.f, d1 = 0.f, d2 = 0.f, dinv = 0.f;
  bool need_sh = false;
  if (touched) {
    const float m0 = means[3 * i], m1 = means[3 * i + 1], m2 = means[3 * i + 2];
    const float *R = cam.R;
    const float tx = fmaf(R[0], m0, fmaf(R[1], m1, fmaf(R[2], m2, cam.t[0])));
    const float ty = fmaf(R[3], m0, fmaf(R[4], m1, fmaf(R[5], m2, cam.t[1])));
    const float tz = fmaf(R[6], m0, fmaf(R[7], m1, fmaf(R[8], m2, cam.t[2])));
    const float o = opac[i];
    const float tau = 2.0f * logf(255.0f * o);
    const float4 q4 = quats[i];
    const float qn2 = q4.x * q4.x + q4.y * q4.y + q4.z * q4.z + q4.w * q4.w;
    if (tz > cam.znear && tau > 0.0f && qn2 > 0.0f) {
      const float qi = 1.0f / sqrtf(qn2);
      const float w = q4.x * qi, x = q4.y * qi, y = q4.z * qi, z = q4.w * qi;
      float rq[3][3] = {{1.f - 2.f * (y * y + z * z), 2.f * (x * y - w * z), 2.f * (x * z + w * y)},
                        {2.f * (x * y + w * z), 1.f - 2.f * (x * x + z * z), 2.f * (y * z - w * x)},
                        {2.f * (x * z - w * y), 2.f * (y * z + w * x), 1.f - 2.f * (x * x + y * y)}};
      const float sc[3] = {expf(log_scales[3 * i]), expf(log_scales[3 * i + 1]),
                           expf(log_scales[3 * i + 2])};
      // M = R (Rq S), u and v the rows of J M (as in the forward pass)
      float M[3][3];
#pragma unroll
      for (int r = 0; r < 3; r++)
#pragma unroll
        for (int c = 0; c < 3; c++)
          M[r][c] = (R[3 * r] * rq[0][c] + R[3 * r + 1] * rq[1][c] + R[3 * r + 2] * rq[2][c]) * sc[c];
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
      const float det = (cx0 * cx0 + cx1 * cx1 + cx2 * cx2) + lp * (uu + vv) + lp * lp;
      if (det > 0.0f) {
        const float idet = 1.0f / det;
        const float ca = syy * idet, cb = -uv * idet, cc = sxx * idet;
        const float gmx = gsp[0], gmy = gsp[1], ga = gsp[2], gb = gsp[3], gc = gsp[4];
        // conic -> Sigma': dL/dSigma' = -Lambda G Lambda, G = [[ga, gb/2], [gb/2, gc]]
        const float p00 = fmaf(ca, ga, 0.5f * cb * gb), p01 = fmaf(0.5f * ca, gb, cb * gc);
        const float p10 = fmaf(cb, ga, 0.5f * cc * gb), p11 = fmaf(0.5f * cb, gb, cc * gc);
        const float dsxx = -fmaf(p00, ca, p01 * cb);
        const float duv = -2.0f * fmaf(p00, cb, p01 * cc);
        const float dsyy = -fmaf(p10, cb, p11 * cc);
        // Sigma' -> u, v -> M and t
        float dM[3][3];
        float sx = 0.f, sy = 0.f, sz = 0.f;
#pragma unroll
        for (int c = 0; c < 3; c++) {
          const float du = fmaf(2.0f * dsxx, u[c], duv * v[c]);
          const float dv = fmaf(2.0f * dsyy, v[c], duv * u[c]);
          dM[0][c] = fxz * du;
          dM[1][c] = fyz * dv;
          dM[2][c] = -(fxz * ux * du + fyz * uy * dv);
          sx = fmaf(du, M[2][c], sx);
          sy = fmaf(dv, M[2][c], sy);
          sz += du * (fxz * ux * M[2][c] - u[c]) + dv * (fyz * uy * M[2][c] - v[c]);
        }
        const float dtx = fxz * (gmx - iz * sx);
        const float dty = fyz * (gmy - iz * sy);
        const float dtz = iz * sz - gmx * fxz * ux - gmy * fyz * uy;
        // M = R A -> A = Rq S -> scales and rotation entries
        float dRq[3][3];
#pragma unroll
        for (int c = 0; c < 3; c++) {
          float ds = 0.f;
#pragma unroll
          for (int r = 0; r < 3; r++) {
            const float dA = R[r] * dM[0][c] + R[3 + r] * dM[1][c] + R[6 + r] * dM[2][c];
            ds = fmaf(dA, rq[r][c], ds);
            dRq[r][c] = dA * sc[c];
          }
          dls[c] = ds * sc[c];
        }
        // rotation entries -> unit quaternion -> quaternion
        const float gw = 2.f * (-z * dRq[0][1] + y * dRq[0][2] + z * dRq[1][0] - x * dRq[1][2] -
                                y * dRq[2][0] + x * dRq[2][1]);
        const float gx = 2.f * (y * dRq[0][1] + z * dRq[0][2] + y * dRq[1][0] - 2.f * x * dRq[1][1] -
                                w * dRq[1][2] + z * dRq[2][0] + w * dRq[2][1] - 2.f * x * dRq[2][2]);
        const float gy = 2.f * (-2.f * y * dRq[0][0] + x * dRq[0][1] + w * dRq[0][2] + x * dRq[1][0] +
                                z * dRq[1][2] - w * dRq[2][0] + z * dRq[2][1] - 2.f * y * dRq[2][2]);
        const float gz = 2.f * (-2.f * z * dRq[0][0] - w * dRq[0][1] + x * dRq[0][2] + w * dRq[1][0] -
                                2.f * z * dRq[1][1] + y * dRq[1][2] + x * dRq[2][0] + y * dRq[2][1]);
        const float qd = w * gw + x * gx + y * gy + z * gz;
        gq = make_float4((gw - w * qd) * qi, (gx - x * qd) * qi, (gy - y * qd) * qi,
                         (gz - z * qd) * qi);
        gop = gsp[5];
        // t = R mu + t_cam
        g0 = R[0] * dtx + R[3] * dty + R[6] * dtz;
        g1 = R[1] * dtx + R[4] * dty + R[7] * dtz;
        g2 = R[2] * dtx + R[5] * dty + R[8] * dtz;
        d0 = m0 - cam.centre[0]; d1 = m1 - cam.centre[1]; d2 = m2 - cam.centre[2];
        const float dn2 = d0 * d0 + d1 * d1 + d2 * d2;
        if (dn2 > 0.0f) {
          dinv = 1.0f / sqrtf(dn2);
          d0 *= dinv; d1 *= dinv; d2 *= dinv;
          need_sh = true;
        }
      }
    }
  }
  // colour: dL/ds_k = Y_k(d) dL/dc, and the view direction's share of dL/dmu
  float buf[K * 3], row[K * 3];
  read_sh<K>(sh, i, need_sh, buf, lds_wave);
#pragma unroll
  for (int j = 0; j < K * 3; j++) row[j] = 0.0f;
  if (need_sh) {
    const float gr = gsp[6], gg = gsp[7], gbl = gsp[8];
    float Y[16], wk[16];
    sh_eval(K, d0, d1, d2, Y);
#pragma unroll
    for (int k = 0; k < K; k++) {
      wk[k] = fmaf(buf[3 * k], gr, fmaf(buf[3 * k + 1], gg, buf[3 * k + 2] * gbl));
      row[3 * k] = Y[k] * gr;
      row[3 * k + 1] = Y[k] * gg;
      row[3 * k + 2] = Y[k] * gbl;
    }
    float e0 = 0.f, e1 = 0.f, e2 = 0.f;
    sh_grad_acc(K, d0, d1, d2, wk, e0, e1, e2);
    const float ed = e0 * d0 + e1 * d1 + e2 * d2;
    g0 = fmaf(e0 - d0 * ed, dinv, g0);
    g1 = fmaf(e1 - d1 * ed, dinv, g1);
    g2 = fmaf(e2 - d2 * ed, dinv, g2);
  }
  if (i < n && acc) {  // another view's share of the same Gaussians' gradients
    gmeans[3 * i] += g0;
    gmeans[3 * i + 1] += g1;
    gmeans[3 * i + 2] += g2;
    gls[3 * i] += dls[0];
    gls[3 * i + 1] += dls[1];
    gls[3 * i + 2] += dls[2];
    const float4 o4 = gquats[i];
    gquats[i] = make_float4(o4.x + gq.x, o4.y + gq.y, o4.z + gq.z, o4.w + gq.w);
    gopac[i] += gop;
  } else if (i < n) {
    gmeans[3 * i] = g0;
    gmeans[3 * i + 1] = g1;
    gmeans[3 * i + 2] = g2;
    gls[3 * i] = dls[0];
    gls[3 * i + 1] = dls[1];
    gls[3 * i + 2] = dls[2];
    gquats[i] = gq;
    gopac[i] = gop;
  }
  // every SH gradient row is written (zeros for culled and untouched Gaussians)
  if constexpr (RO::V > 0) {
    const int lane = threadIdx.x & 63;
    const int w0 = i - lane;
    if (w0 < n) {
      wave_sync();  // the LDS rows read above are reused
#pragma unroll
      for (int j = 0; j < RO::V; j++)
        lds_wave[lane * RO::SV + j] =
            make_uint4(__float_as_uint(row[4 * j]), __float_as_uint(row[4 * j + 1]),
                       __float_as_uint(row[4 * j + 2]), __float_as_uint(row[4 * j + 3]));
      stage_rows_out<RO::V, RO::SV>(reinterpret_cast<uint4 *>(gsh) + (size_t)w0 * RO::V,
                                    min(64, n - w0), lds_wave, lane, acc);
    }
  } else if (i < n) {
    float *gsh_i = gsh + (size_t)i * (K * 3);
#pragma unroll
    for (int j = 0; j < K * 3; j++) gsh_i[j] = acc ? gsh_i[j] + row[j] : row[j];
  }
}

template <typename ShT>
hipError_t launch_project_bwd(int n, const float *means, const float *log_scales,
                              const float *quats, const float *opac, const ShT *sh, int degree,
                              const CamK &cam, const float *dsplat, float *gmeans, float *gls,
                              float *gquats, float *gopac, float *gsh, bool acc, hipStream_t st) {
  if (n == 0) return hipSuccess;
  dim3 grid(gs_div_up(n, 256)), block(256);
  const float4 *q4 = reinterpret_cast<const float4 *>(quats);
  float4 *gq4 = reinterpret_cast<float4 *>(gquats);
  switch (degree) {
    case 0: hipLaunchKernelGGL((k_project_bwd<1, ShT>), grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, dsplat, gmeans, gls, gq4, gopac, gsh, acc); break;
    case 1: hipLaunchKernelGGL((k_project_bwd<4, ShT>), grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, dsplat, gmeans, gls, gq4, gopac, gsh, acc); break;
    case 2: hipLaunchKernelGGL((k_project_bwd<9, ShT>), grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, dsplat, gmeans, gls, gq4, gopac, gsh, acc); break;
    default: hipLaunchKernelGGL((k_project_bwd<16, ShT>), grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, dsplat, gmeans, gls, gq4, gopac, gsh, acc); break;
  }
  return hipGetLastError();
}

template <typename ShT>
hipError_t launch_project(int n, const float *means, const float *log_scales, const float *quats,
                          const float *opac, const ShT *sh, int degree, const CamK &cam,
                          float *splats, hipStream_t st) {
  if (n == 0) return hipSuccess;
  dim3 grid(gs_div_up(n, 256)), block(256);
  const float4 *q4 = reinterpret_cast<const float4 *>(quats);
  Splat *out = reinterpret_cast<Splat *>(splats);
  switch (degree) {
    case 0: hipLaunchKernelGGL((k_project<1, ShT>), grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, out); break;
    case 1: hipLaunchKernelGGL((k_project<4, ShT>), grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, out); break;
    case 2: hipLaunchKernelGGL((k_project<9, ShT>), grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, out); break;
    default: hipLaunchKernelGGL((k_project<16, ShT>), grid, block, 0, st, n, means, log_scales, q4, opac, sh, cam, out); break;
  }
  return hipGetLastError();
}

}  // namespace

// SH stored as fp32 (sh_bf16 == false) or as bf16 bits (true).
hipError_t gs_launch_project(int n, const float *means, const float *log_scales, const float *quats,
                             const float *opac, const void *sh, bool sh_bf16, int degree,
                             const CamK &cam, float *splats, hipStream_t st) {
  return sh_bf16 ? launch_project(n, means, log_scales, quats, opac,
                                  static_cast<const uint16_t *>(sh), degree, cam, splats, st)
                 : launch_project(n, means, log_scales, quats, opac, static_cast<const float *>(sh),
                                  degree, cam, splats, st);
}

hipError_t gs_launch_project_bwd(int n, const float *means, const float *log_scales,
                                 const float *quats, const float *opac, const void *sh,
                                 bool sh_bf16, int degree, const CamK &cam, const float *dsplat,
                                 float *gmeans, float *gls, float *gquats, float *gopac,
                                 float *gsh, bool acc, hipStream_t st) {
  return sh_bf16 ? launch_project_bwd(n, means, log_scales, quats, opac,
                                      static_cast<const uint16_t *>(sh), degree, cam, dsplat,
                                      gmeans, gls, gquats, gopac, gsh, acc, st)
                 : launch_project_bwd(n, means, log_scales, quats, opac,
                                      static_cast<const float *>(sh), degree, cam, dsplat, gmeans,
                                      gls, gquats, gopac, gsh, acc, st);
}
