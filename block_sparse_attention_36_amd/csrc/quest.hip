// Quest backbone tile scores: per query row the largest q.k over each key block's
// coordinate box [k_min, k_max], and per tile the maximum over its query rows
// ("Uncertainty-gated selection for block-sparse attention", technical summary,
// Methodology steps 1-2: per-coordinate upper bounds from K-min/K-max as a scoring
// backbone; a tile's score is the maximum over its rows).
//
// sum_d max(q_d kmin_d, q_d kmax_d) = q+ . kmax + q- . kmin with q+ = max(q, 0) and
// q- = min(q, 0), so a row's bounds against a run of key blocks are one contraction
// of [q+ | q-] (length 2D) with [kmax | kmin], done on the bf16 matrix cores
// (V_MFMA_F32_32X32X16_BF16).  bf16 queries split exactly into q+ and q-; E4M3
// query codes decode exactly to bf16 and their (non-negative) scale multiplies the
// tile's result.  Bounds of bf16 keys are bf16 values, so every product is exact
// and only the fp32 accumulation rounds.  Bounds of E4M3 keys (code times scale)
// are split into a bf16 head and tail, x = hi + lo with |x - hi - lo| <= 2^-18 |x|,
// and the contraction runs over [q+ | q- | q+ | q-] . [max_hi | min_hi | max_lo |
// min_lo].
//
// Work: one workgroup per (selection unit, query tile) with B/32 waves; wave w holds
// query rows [32w, 32w+32) of the tile as A fragments in registers.  Key blocks
// 0..i go by in chunks of 32: each chunk's packed bounds (32 rows of NP*D bf16,
// rows padded by 16 bytes so the per-lane 16-byte reads of one MFMA operand spread
// over the LDS banks) are staged in LDS, double-buffered, the next chunk's global
// loads in flight while the current one is contracted.  The maximum over a wave's
// valid rows, then over the waves, gives the chunk's 32 tile scores.  Per-group
// units loop over the group's heads and keep the running maximum in the output.
// Workgroups go kv-head major, the longest tiles first, and the units of one kv
// head at one tile on one XCD (workgroup id mod 8), whose L2 then holds their
// common bounds.
#include <atomic>

#include "common.h"
#include "launch.h"

namespace bsa {

namespace {

// f32 bounds [Hkv, nb, D] (min and max) -> packed bf16 rows [Hkv, nb, NP*D]:
// [max_hi | min_hi] (NP = 2) or [max_hi | min_hi | max_lo | min_lo] (NP = 4).
// One thread per 8 consecutive coordinates of one block row.
__global__ __launch_bounds__(256) void quest_pack_kernel(const float* __restrict__ kmin,
                                                         const float* __restrict__ kmax,
                                                         unsigned* __restrict__ packed,
                                                         int64_t rows, int D, int NP) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = D / 8;
  if (idx >= rows * per_row) return;
  const int64_t row = idx / per_row;
  const int d = (int)(idx % per_row) * 8;
  const float* src[2] = {kmax + row * D + d, kmin + row * D + d};
  unsigned* dst = packed + (row * NP * D) / 2;  // two bf16 per dword
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const f32x4 x0 = *(const f32x4*)src[part], x1 = *(const f32x4*)(src[part] + 4);
    const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    u32x4 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
      const float h0 = __uint_as_float(hi[e] << 16), h1 = __uint_as_float(hi[e] & 0xFFFF0000u);
      lo[e] = pack_bf16x2(x[2 * e] - h0, x[2 * e + 1] - h1);  // the differences are exact
    }
    *(u32x4*)(dst + (part * D + d) / 2) = hi;
    if (NP == 4) *(u32x4*)(dst + ((2 + part) * D + d) / 2) = lo;
  }
}

struct QuestArgs {
  const void* q;
  const float* q_scale;
  const unsigned short* packed;
  float* scores;
  int64_t S;
  int Hq, Hkv, nb, per_group;
};

template <int D, int B, int NP>
struct QCfg {
  static constexpr int NW = B / 32;           // waves per workgroup
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int NS = D / 16;           // contraction steps per D
  static constexpr int KSTEPS = NP * NS;      // steps per chunk
  static constexpr int ROW = NP * D * 2;      // packed bytes per key block
  static constexpr int LROW = ROW + 16;       // padded LDS row
  static constexpr int CH = 32;               // key blocks per chunk
  static constexpr int BUF = CH * LROW;       // bytes per LDS buffer
  static constexpr int PIECES = CH * ROW / 16;
  static constexpr int PPT = PIECES / NT;     // 16-byte pieces per thread per chunk
  static_assert(PIECES % NT == 0, "chunk pieces must divide among the threads");
};

// 0xFFFF in each bf16 half of x whose sign bit is set: x & m is the non-positive
// part of the pair, x & ~m the non-negative part
__device__ __forceinline__ unsigned neg_mask(unsigned x) {
  return ((x >> 15) & 0x00010001u) * 0xFFFFu;
}

// HP heads of one kv head per workgroup pass: every bounds fragment read from LDS
// feeds HP products, and the chunk staging and barrier serve HP heads.
template <int D, int B, bool FP8, int NP, int HP>
__global__ __launch_bounds__(64 * (B / 32), 2) void quest_score_kernel(QuestArgs a) {
  typedef QCfg<D, B, NP> C;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float* red = (float*)(lds + 2 * C::BUF);  // [2][NW][HP][32]
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / a.Hkv, nb = a.nb;
  const int Gu = a.per_group ? 1 : G / HP;  // workgroups per (kv head, query block)
  const int bid = blockIdx.x;
  const int xcd = bid & 7, t8 = bid >> 3;
  const int hh = t8 % Gu;
  const int r = (t8 / Gu) * 8 + xcd;
  if (r >= a.Hkv * nb) return;  // padding workgroup (uniform: no barrier reached)
  const int g = r / nb, i = nb - 1 - r % nb;
  const int nheads = a.per_group ? G : HP;  // heads this workgroup covers, HP per pass
  const int hbase = a.per_group ? g * G : g * G + hh * HP;
  const int nch = i / C::CH + 1;
  const unsigned char* kp = (const unsigned char*)(a.packed + (size_t)g * nb * NP * D);

  u32x4 pf[C::PPT];
  auto stage_load = [&](int c) {
#pragma unroll
    for (int p = 0; p < C::PPT; ++p) {
      const int piece = p * C::NT + tid;
      const int row = piece / (C::ROW / 16), col = piece % (C::ROW / 16);
      int j = c * C::CH + row;
      j = j < nb ? j : nb - 1;  // rows past the last block are loaded but never used
      pf[p] = *(const u32x4*)(kp + (size_t)j * C::ROW + col * 16);
    }
  };
  auto stage_write = [&](int buf) {
#pragma unroll
    for (int p = 0; p < C::PPT; ++p) {
      const int piece = p * C::NT + tid;
      const int row = piece / (C::ROW / 16), col = piece % (C::ROW / 16);
      *(u32x4*)(lds + buf * C::BUF + row * C::LROW + col * 16) = pf[p];
    }
  };

  for (int hx = 0; hx < nheads; hx += HP) {
    if (hx > 0) __syncthreads();  // the previous pass's last reduction has read red[]
    // A fragments: row (l & 31) of this wave's 32, coordinates 16s + 8(l >> 5) + [0, 8)
    const int64_t t = (int64_t)i * B + wave * 32 + (l & 31);
    const bool rv = t < a.S;
    u32x4 qp[HP][C::NS], qn[HP][C::NS];
    float qs[HP];
#pragma unroll
    for (int hp = 0; hp < HP; ++hp) {
      const int h = hbase + hx + hp;
      qs[hp] = FP8 ? a.q_scale[(size_t)h * nb + i] : 1.0f;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const int d0 = 16 * s + 8 * (l >> 5);
        u32x4 x = u32x4{0u, 0u, 0u, 0u};
        if (rv) {
          const size_t e0 = ((size_t)t * a.Hq + h) * D + d0;
          if (FP8) {
            const u32x2 c8 = *(const u32x2*)((const unsigned char*)a.q + e0);
            const u32x2 lo = e4m3x4_to_bf16x4(c8[0]), hi = e4m3x4_to_bf16x4(c8[1]);
            x = u32x4{lo[0], lo[1], hi[0], hi[1]};
          } else {
            x = *(const u32x4*)((const unsigned char*)a.q + e0 * 2);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned m = neg_mask(x[e]);
          qn[hp][s][e] = x[e] & m;
          qp[hp][s][e] = x[e] & ~m;
        }
      }
    }

    stage_load(0);
    stage_write(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      const int cur = c & 1;
      if (c + 1 < nch) stage_load(c + 1);
      // bf16 bounds: two accumulators per head (even and odd contraction steps),
      // independent product chains; the split bounds' longer contraction keeps one
      constexpr int NA = NP == 2 ? 2 : 1;
      f32x16 accs[HP][NA];
#pragma unroll
      for (int hp = 0; hp < HP; ++hp)
#pragma unroll
        for (int q = 0; q < NA; ++q) accs[hp][q] = f32x16{0};
      const unsigned char* bb = lds + cur * C::BUF + (l & 31) * C::LROW + 16 * (l >> 5);
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const u32x4 bf = *(const u32x4*)(bb + 32 * s);
#pragma unroll
        for (int hp = 0; hp < HP; ++hp) {
          const u32x4 af = ((s / C::NS) & 1) ? qn[hp][s % C::NS] : qp[hp][s % C::NS];
          accs[hp][s % NA] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, af), __builtin_bit_cast(bf16x8, bf), accs[hp][s % NA], 0,
              0, 0);
        }
      }
      // maximum over this wave's valid rows, for column (block) 32c + (l & 31)
#pragma unroll
      for (int hp = 0; hp < HP; ++hp) {
        f32x16 acc = accs[hp][0];
#pragma unroll
        for (int q = 1; q < NA; ++q) acc += accs[hp][q];
        float m = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = (e >> 2) * 8 + (l >> 5) * 4 + (e & 3);
          if ((int64_t)i * B + wave * 32 + row < a.S) m = fmaxf(m, acc[e]);
        }
        m = max_with_other_half(m);
        if (l < 32) red[((cur * C::NW + wave) * HP + hp) * 32 + l] = m;
      }
      if (c + 1 < nch) stage_write(cur ^ 1);
      __syncthreads();
      // wave hp (< HP) finishes head hp; a per-group row takes the maximum over
      // all G heads: over the pass's heads through LDS, over passes in memory
      const int j = c * C::CH + l;
      if (wave < HP && l < 32 && j <= i) {
        const int hp = wave;
        float v = red[(cur * C::NW * HP + hp) * 32 + l];
#pragma unroll
        for (int w = 1; w < C::NW; ++w) v = fmaxf(v, red[((cur * C::NW + w) * HP + hp) * 32 + l]);
        v *= qs[hp];
        if (!a.per_group) {
          a.scores[((size_t)(hbase + hx + hp) * nb + i) * nb + j] = v;
        } else if (HP == 1) {
          float* srow = a.scores + ((size_t)g * nb + i) * nb;
          srow[j] = hx == 0 ? v : fmaxf(srow[j], v);
        } else {
          red[(2 * C::NW * HP + hp) * 32 + l] = v;
        }
      }
      if (HP > 1 && a.per_group) {
        __syncthreads();
        if (wave == 0 && l < 32 && j <= i) {
          float v = red[(2 * C::NW * HP) * 32 + l];
#pragma unroll
          for (int hp = 1; hp < HP; ++hp) v = fmaxf(v, red[(2 * C::NW * HP + hp) * 32 + l]);
          float* srow = a.scores + ((size_t)g * nb + i) * nb;
          srow[j] = hx == 0 ? v : fmaxf(srow[j], v);
        }
      }
    }
  }
}

template <int D, int B, bool FP8, int NP, int HP>
hipError_t launch_quest_t(const Shape& sh, const QuestArgs& a, hipStream_t stream) {
  typedef QCfg<D, B, NP> C;
  auto kern = quest_score_kernel<D, B, FP8, NP, HP>;
  constexpr int lds_bytes = 2 * C::BUF + (2 * C::NW * HP + HP) * 32 * 4;
  static_assert(lds_bytes <= 80 * 1024, "LDS budget");
  // the LDS limit is raised once per device (64 KiB and more need the attribute)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int Gu = sh.per_group ? 1 : sh.G() / HP;
  const int64_t rows8 = ((int64_t)sh.Hkv * sh.nb + 7) / 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rows8 * 8 * Gu)), dim3(C::NT), lds_bytes, stream, a);
  return hipGetLastError();
}

template <int D, int B>
hipError_t launch_quest_db(const Shape& sh, const QuestArgs& a, hipStream_t stream) {
#ifndef BSA_QUEST_HP
#define BSA_QUEST_HP 2
#endif
  // two heads per pass wherever the group size allows (at B = 64 the staging
  // registers of the two-wave workgroup leave no room for the second head)
  if (BSA_QUEST_HP == 2 && B == 128 && sh.G() % 2 == 0)
    return sh.fp8 ? launch_quest_t<D, B, true, 4, 2>(sh, a, stream)
                  : launch_quest_t<D, B, false, 2, 2>(sh, a, stream);
  return sh.fp8 ? launch_quest_t<D, B, true, 4, 1>(sh, a, stream)
                : launch_quest_t<D, B, false, 2, 1>(sh, a, stream);
}

}  // namespace

size_t quest_workspace_bytes(const Shape& sh) {
  const size_t np = sh.fp8 ? 4 : 2;
  return ((size_t)sh.Hkv * sh.nb * np * sh.D * 2 + 255) & ~(size_t)255;
}

hipError_t launch_quest_scores(const Shape& sh, const void* q, const float* q_scale,
                               const float* k_min, const float* k_max, float* scores,
                               void* workspace, hipStream_t stream) {
  const int np = sh.fp8 ? 4 : 2;
  const int64_t rows = (int64_t)sh.Hkv * sh.nb;
  const int64_t threads = rows * (sh.D / 8);
  hipLaunchKernelGGL(quest_pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, k_min, k_max, (unsigned*)workspace, rows, sh.D, np);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  QuestArgs a;
  a.q = q;
  a.q_scale = q_scale;
  a.packed = (const unsigned short*)workspace;
  a.scores = scores;
  a.S = sh.S;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.nb = sh.nb;
  a.per_group = sh.per_group;
  if (sh.D == 128)
    return sh.B == 128 ? launch_quest_db<128, 128>(sh, a, stream)
                       : launch_quest_db<128, 64>(sh, a, stream);
  return sh.B == 128 ? launch_quest_db<64, 128>(sh, a, stream)
                     : launch_quest_db<64, 64>(sh, a, stream);
}

}  // namespace bsa
