// Block pooling: query/key block centroids, query-centroid norms, key-block radii.
//
// Method: keys are grouped into blocks of B tokens and each block is represented
// by its mean ("Uncertainty-gated selection for block-sparse attention", technical
// summary, Methodology step 1: mean-pooling backbone); the rescue branch needs a
// per-(prompt, layer, head) key-block radius (RBS-Attention, third and fourth
// paragraphs), here the largest distance of a key from its block mean.
//
// Design: HBM-bound streaming reduction.  Each thread owns 8 consecutive elements
// of the [H*D] token row, so every row load is one contiguous, fully coalesced
// 16-byte (bf16) or 8-byte (E4M3) access per thread.  Queries: one workgroup per
// (token block, chunk of heads), rows loaded eight at a time.  Keys (far fewer
// heads): eight waves per block split its rows, which stay in registers for the
// radius pass.
//
// Key-block bounds (the Quest backbone's summary, same page, Methodology step 1:
// per-coordinate upper bounds from K-min/K-max): the coordinate-wise minimum and
// maximum of each block's dequantised keys, with the same row split as the key
// centroids.
#include "common.h"
#include "launch.h"

namespace bsa {

namespace {

template <bool FP8>
struct RowLoad;

template <>
struct RowLoad<false> {  // 8 bf16
  typedef u32x4 raw;
  static __device__ __forceinline__ raw load(const void* p) { return *(const u32x4*)p; }
  static __device__ __forceinline__ void add(float* acc, const raw& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(v[e] << 16);
      acc[2 * e + 1] += __uint_as_float(v[e] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void decode(float* x, const raw& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(v[e] << 16);
      x[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
    }
  }
  static constexpr int elem_bytes = 2;
};

template <>
struct RowLoad<true> {  // 8 E4M3 codes
  typedef u32x2 raw;
  static __device__ __forceinline__ raw load(const void* p) { return *(const u32x2*)p; }
  static __device__ __forceinline__ void decode(float* x, const raw& v) {
    const f32x4 a = e4m3x4_to_f32x4(v[0]), b = e4m3x4_to_f32x4(v[1]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
  }
  static __device__ __forceinline__ void add(float* acc, const raw& v) {
    float x[8];
    decode(x, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[e];
  }
  static constexpr int elem_bytes = 1;
};

// Query rows: one 16-byte load per row and thread, so 8 bf16 or 16 E4M3 codes.
template <bool FP8>
struct QLoad;

template <>
struct QLoad<false> : RowLoad<false> {
  static constexpr int EPT = 8;
  static constexpr int BATCH = 8;
};

template <>
struct QLoad<true> {  // 16 E4M3 codes
  typedef u32x4 raw;
  static constexpr int EPT = 16;
  // 16 rows in flight: a 128K-token layer of 32 heads has only four waves per
  // SIMD to pool with (2 % faster than 8 there; no gain for bf16)
  static constexpr int BATCH = 16;
  static constexpr int elem_bytes = 1;
  static __device__ __forceinline__ raw load(const void* p) { return *(const u32x4*)p; }
  static __device__ __forceinline__ void add(float* acc, const raw& v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = e4m3x4_to_f32x4(v[q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * q + e] += x[e];
    }
  }
};

// Sum of `cnt` rows (row_bytes apart) of the elements one load of L covers at base.
// Rows are loaded L::BATCH at a time, the loads issued together, then added in
// row order.
template <class L>
__device__ __forceinline__ void sum_rows(const unsigned char* base, size_t row_bytes, int cnt,
                                         float* acc) {
  constexpr int NBT = L::BATCH;
  int t = 0;
  for (; t + NBT <= cnt; t += NBT) {
    typename L::raw v[NBT];
#pragma unroll
    for (int u = 0; u < NBT; ++u) v[u] = L::load(base + (size_t)(t + u) * row_bytes);
#pragma unroll
    for (int u = 0; u < NBT; ++u) L::add(acc, v[u]);
  }
  for (; t < cnt; ++t) L::add(acc, L::load(base + (size_t)t * row_bytes));
}

// Sum over the D/EPT consecutive lanes that hold one head's row.
template <int D, int EPT>
__device__ __forceinline__ float head_lane_sum(float x) {
#pragma unroll
  for (int o = D / (2 * EPT); o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <bool FP8, int D>
__global__ void pool_q_kernel(const void* __restrict__ q, const float* __restrict__ q_scale,
                              float* __restrict__ qc, float* __restrict__ qn, int64_t S, int Hq,
                              int Hkv, int B, int nb, int per_group, int HW) {
  extern __shared__ float red[];  // [HW][D], per-head means for the group sum
  typedef QLoad<FP8> L;
  constexpr int EPT = L::EPT;
  const int i = blockIdx.x;
  const int h0 = blockIdx.y * HW;
  const int tid = threadIdx.x;
  const int hl = (tid * EPT) / D, d = (tid * EPT) % D;
  const int h = h0 + hl;
  const bool active = h < Hq;
  const int64_t t0 = (int64_t)i * B;
  const int cnt = (int)((S - t0) < B ? (S - t0) : B);
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  if (active) {
    const size_t row_bytes = (size_t)Hq * D * L::elem_bytes;
    const unsigned char* base = (const unsigned char*)q + (size_t)t0 * row_bytes +
                                ((size_t)h * D + d) * L::elem_bytes;
    sum_rows<L>(base, row_bytes, cnt, acc);
  }
  const float mul = (FP8 && active ? q_scale[(size_t)h * nb + i] : 1.0f) / (float)cnt;
  float mean[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) mean[e] = acc[e] * mul;

  if (!per_group) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) ss += mean[e] * mean[e];
    ss = head_lane_sum<D, EPT>(ss);
    if (active) {
      float* dst = qc + ((size_t)h * nb + i) * D + d;
#pragma unroll
      for (int e = 0; e < EPT; e += 4)
        *(f32x4*)(dst + e) = f32x4{mean[e], mean[e + 1], mean[e + 2], mean[e + 3]};
      if (qn && d == 0) qn[(size_t)h * nb + i] = sqrtf(ss);
    }
    return;
  }
  // per-group rows: mean over the group's heads of the per-head means
  const int G = Hq / Hkv;
#pragma unroll
  for (int e = 0; e < EPT; ++e) red[hl * D + d + e] = mean[e];
  __syncthreads();
  const int ul = hl;  // this thread now works for local unit ul (if any)
  const int u = h0 / G + ul;
  const bool uact = ul < HW / G && u < Hkv;
  float gm[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) gm[e] = 0.f;
  if (uact) {
    for (int gg = 0; gg < G; ++gg) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) gm[e] += red[(ul * G + gg) * D + d + e];
    }
  }
  const float invg = 1.0f / (float)G;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    gm[e] *= invg;
    ss += gm[e] * gm[e];
  }
  ss = head_lane_sum<D, EPT>(ss);
  if (uact) {
    float* dst = qc + ((size_t)u * nb + i) * D + d;
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *(f32x4*)(dst + e) = f32x4{gm[e], gm[e + 1], gm[e + 2], gm[e + 3]};
    if (qn && d == 0) qn[(size_t)u * nb + i] = sqrtf(ss);
  }
}

// Key blocks: one workgroup of KW waves per (key block, chunk of kv heads).
// Wave w owns rows [w*R, (w+1)*R) of the block (R = B / KW) and keeps them in
// registers, so the radius pass reuses them instead of reading the block again;
// partial sums and maxima meet in LDS.  KW * R rows are in flight per
// workgroup, enough to keep HBM busy with only nb workgroups.
template <bool FP8, int D, int KW, int R>
__global__ __launch_bounds__(64 * KW) void pool_k_kernel(
    const void* __restrict__ k, const float* __restrict__ k_scale, float* __restrict__ kc,
    float* __restrict__ kr, int64_t S, int Hkv, int B, int nb, int HW) {
  typedef RowLoad<FP8> L;
  __shared__ f32x4 part[KW][64][2];
  __shared__ float pmax[KW][64];
  const int j = blockIdx.x;
  const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gl = (l * 8) / D, d = (l * 8) % D;
  const int g = blockIdx.y * HW + gl;
  const bool active = gl < HW && g < Hkv;
  const int64_t t0 = (int64_t)j * B;
  const int cnt = (int)((S - t0) < B ? (S - t0) : B);
  const size_t row_bytes = (size_t)Hkv * D * L::elem_bytes;
  const unsigned char* base = (const unsigned char*)k + (size_t)t0 * row_bytes +
                              ((size_t)(active ? g : 0) * D + d) * L::elem_bytes;
  const int r0 = w * R;
  typename L::raw v[R];
#pragma unroll
  for (int u = 0; u < R; ++u)
    if (active && r0 + u < cnt) v[u] = L::load(base + (size_t)(r0 + u) * row_bytes);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < R; ++u)
    if (active && r0 + u < cnt) L::add(acc, v[u]);
  part[w][l][0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  part[w][l][1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  __syncthreads();
  // every wave forms the same mean (fixed summation order over the waves)
  float sum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int ww = 0; ww < KW; ++ww) {
    const f32x4 a0 = part[ww][l][0], a1 = part[ww][l][1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sum[e] += a0[e];
      sum[4 + e] += a1[e];
    }
  }
  const float scale = (FP8 && active) ? k_scale[(size_t)g * nb + j] : 1.0f;
  const float mul = scale / (float)cnt;
  float c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = sum[e] * mul;
  if (w == 0 && active) {
    float* dst = kc + ((size_t)g * nb + j) * D + d;
    *(f32x4*)dst = f32x4{c[0], c[1], c[2], c[3]};
    *(f32x4*)(dst + 4) = f32x4{c[4], c[5], c[6], c[7]};
  }
  if (!kr) return;  // uniform: no barrier follows for anyone
  // largest distance of this wave's rows from the mean
  float mx = 0.f;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    float pt = 0.f;
    if (active && r0 + u < cnt) {
      float x[8];
      L::decode(x, v[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float df = x[e] * scale - c[e];
        pt += df * df;
      }
    }
    pt = head_lane_sum<D, 8>(pt);
    mx = fmaxf(mx, pt);
  }
  pmax[w][l] = mx;
  __syncthreads();
  if (w == 0 && active && d == 0) {
    float m = 0.f;
#pragma unroll
    for (int ww = 0; ww < KW; ++ww) m = fmaxf(m, pmax[ww][l]);
    kr[(size_t)g * nb + j] = sqrtf(m);
  }
}

// Coordinate-wise minimum and maximum of each key block (dequantised values), one
// workgroup of KW waves per (key block, chunk of kv heads), wave w over rows
// [w*R, (w+1)*R); the per-wave extremes meet in LDS.
template <bool FP8, int D, int KW, int R>
__global__ __launch_bounds__(64 * KW) void kbounds_kernel(
    const void* __restrict__ k, const float* __restrict__ k_scale, float* __restrict__ kmin,
    float* __restrict__ kmax, int64_t S, int Hkv, int B, int nb, int HW) {
  typedef RowLoad<FP8> L;
  __shared__ f32x4 pmin[KW][64][2];
  __shared__ f32x4 pmax[KW][64][2];
  const int j = blockIdx.x;
  const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gl = (l * 8) / D, d = (l * 8) % D;
  const int g = blockIdx.y * HW + gl;
  const bool active = gl < HW && g < Hkv;
  const int64_t t0 = (int64_t)j * B;
  const int cnt = (int)((S - t0) < B ? (S - t0) : B);
  const size_t row_bytes = (size_t)Hkv * D * L::elem_bytes;
  const unsigned char* base = (const unsigned char*)k + (size_t)t0 * row_bytes +
                              ((size_t)(active ? g : 0) * D + d) * L::elem_bytes;
  const int r0 = w * R;
  const float scale = (FP8 && active) ? k_scale[(size_t)g * nb + j] : 1.0f;
  typename L::raw v[R];
#pragma unroll
  for (int u = 0; u < R; ++u)
    if (active && r0 + u < cnt) v[u] = L::load(base + (size_t)(r0 + u) * row_bytes);
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = INFINITY;
    hi[e] = -INFINITY;
  }
#pragma unroll
  for (int u = 0; u < R; ++u) {
    if (active && r0 + u < cnt) {
      float x[8];
      L::decode(x, v[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = FP8 ? x[e] * scale : x[e];
        lo[e] = fminf(lo[e], y);
        hi[e] = fmaxf(hi[e], y);
      }
    }
  }
  pmin[w][l][0] = f32x4{lo[0], lo[1], lo[2], lo[3]};
  pmin[w][l][1] = f32x4{lo[4], lo[5], lo[6], lo[7]};
  pmax[w][l][0] = f32x4{hi[0], hi[1], hi[2], hi[3]};
  pmax[w][l][1] = f32x4{hi[4], hi[5], hi[6], hi[7]};
  __syncthreads();
  if (w != 0 || !active) return;  // (no barrier follows)
#pragma unroll
  for (int ww = 1; ww < KW; ++ww) {
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      const f32x4 a = pmin[ww][l][hq], b = pmax[ww][l][hq];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[4 * hq + e] = fminf(lo[4 * hq + e], a[e]);
        hi[4 * hq + e] = fmaxf(hi[4 * hq + e], b[e]);
      }
    }
  }
  const size_t o = ((size_t)g * nb + j) * D + d;
  *(f32x4*)(kmin + o) = f32x4{lo[0], lo[1], lo[2], lo[3]};
  *(f32x4*)(kmin + o + 4) = f32x4{lo[4], lo[5], lo[6], lo[7]};
  *(f32x4*)(kmax + o) = f32x4{hi[0], hi[1], hi[2], hi[3]};
  *(f32x4*)(kmax + o + 4) = f32x4{hi[4], hi[5], hi[6], hi[7]};
}

template <bool FP8, int D>
hipError_t launch_kbounds_t(const Shape& sh, const void* k, const float* k_scale, float* kmin,
                            float* kmax, hipStream_t stream) {
  const int HWK = 512 / D;
  dim3 gk(sh.nb, (sh.Hkv + HWK - 1) / HWK);
  if (sh.B == 128)
    hipLaunchKernelGGL((kbounds_kernel<FP8, D, 8, 16>), gk, dim3(512), 0, stream, k, k_scale,
                       kmin, kmax, sh.S, sh.Hkv, sh.B, sh.nb, HWK);
  else
    hipLaunchKernelGGL((kbounds_kernel<FP8, D, 8, 8>), gk, dim3(512), 0, stream, k, k_scale,
                       kmin, kmax, sh.S, sh.Hkv, sh.B, sh.nb, HWK);
  return hipGetLastError();
}

template <bool FP8, int D>
hipError_t launch_pool_t(const Shape& sh, const void* q, const void* k, const float* q_scale,
                         const float* k_scale, float* q_centroid, float* q_norm,
                         float* k_centroid, float* k_radius, hipStream_t stream) {
  constexpr int EPT = QLoad<FP8>::EPT;
  const int maxh = 256 * EPT / D;  // heads per workgroup at 256 threads
  int HW = sh.Hq < maxh ? sh.Hq : maxh;
  if (sh.per_group) HW = (HW / sh.G()) * sh.G();  // whole groups per workgroup
  dim3 gq(sh.nb, (sh.Hq + HW - 1) / HW);
  hipLaunchKernelGGL((pool_q_kernel<FP8, D>), gq, dim3(HW * D / EPT), HW * D * sizeof(float), stream,
                     q, q_scale, q_centroid, q_norm, sh.S, sh.Hq, sh.Hkv, sh.B, sh.nb,
                     sh.per_group, HW);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // key blocks: 64 threads cover 512 / D heads; eight waves split the block's rows
  const int HWK = 512 / D;
  dim3 gk(sh.nb, (sh.Hkv + HWK - 1) / HWK);
  if (sh.B == 128)
    hipLaunchKernelGGL((pool_k_kernel<FP8, D, 8, 16>), gk, dim3(512), 0, stream, k, k_scale,
                       k_centroid, k_radius, sh.S, sh.Hkv, sh.B, sh.nb, HWK);
  else
    hipLaunchKernelGGL((pool_k_kernel<FP8, D, 8, 8>), gk, dim3(512), 0, stream, k, k_scale,
                       k_centroid, k_radius, sh.S, sh.Hkv, sh.B, sh.nb, HWK);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_key_bounds(const Shape& sh, const void* k, const float* k_scale, float* kmin,
                             float* kmax, hipStream_t stream) {
  if (sh.D == 128)
    return sh.fp8 ? launch_kbounds_t<true, 128>(sh, k, k_scale, kmin, kmax, stream)
                  : launch_kbounds_t<false, 128>(sh, k, k_scale, kmin, kmax, stream);
  return sh.fp8 ? launch_kbounds_t<true, 64>(sh, k, k_scale, kmin, kmax, stream)
                : launch_kbounds_t<false, 64>(sh, k, k_scale, kmin, kmax, stream);
}

hipError_t launch_pool(const Shape& sh, const void* q, const void* k, const float* q_scale,
                       const float* k_scale, float* q_centroid, float* q_norm, float* k_centroid,
                       float* k_radius, hipStream_t stream) {
  if (sh.D == 128)
    return sh.fp8 ? launch_pool_t<true, 128>(sh, q, k, q_scale, k_scale, q_centroid, q_norm,
                                             k_centroid, k_radius, stream)
                  : launch_pool_t<false, 128>(sh, q, k, q_scale, k_scale, q_centroid, q_norm,
                                              k_centroid, k_radius, stream);
  return sh.fp8 ? launch_pool_t<true, 64>(sh, q, k, q_scale, k_scale, q_centroid, q_norm,
                                          k_centroid, k_radius, stream)
                : launch_pool_t<false, 64>(sh, q, k, q_scale, k_scale, q_centroid, q_norm,
                                           k_centroid, k_radius, stream);
}

}  // namespace bsa
