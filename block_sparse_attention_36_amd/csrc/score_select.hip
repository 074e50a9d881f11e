// Block scores, per-row selection, and CSR emission.
//
// Scores: s[u][i][j] = qbar[u][i] . kbar[kv(u)][j], j <= i, the mean-pooling inner
// product ("Uncertainty-gated selection for block-sparse attention", technical
// summary, Methodology step 1).  Computed on the bf16 matrix cores with each fp32
// operand split into two bf16 parts (three products per step), one workgroup per
// 128x128 tile of the causal lower triangle, to within about 3e-6 of
// ||qbar|| ||kbar||.
//
// Selection (one wave per row (u, i)), on the candidates C_i = {0..i} minus the
// forced blocks, ranked by descending score with the lowest index first on ties:
//   top-k  : the first k (same page, Methodology step 2, the kv_idx list), or the
//            first rho*k when the gate fires: p(0) - p(1) < theta for
//            p = softmax(tau*s) over C_i (same page, lay summary "The Solution";
//            Methodology step 5 names rho);
//   base   : the shortest prefix whose softmax mass reaches mu (RBS-Attention, third
//            paragraph, the base branch with its own threshold);
//   rescue : the first ceil(phi*|C_i|) ranked by b = s + ||qbar||*r (RBS-Attention,
//            third and fourth paragraphs, the radius rescue branch);
//   kept   : forced U top-k U base U rescue (the masks are unioned).
// The sigma gate (same page, Methodology steps 3-5) decides per tile instead of
// per row: each row records its cut margin sigma = (s(k-1) - s(k)) / (s(0) - s(k))
// over its sorted candidate scores together with the extra blocks a budget of
// rho*k would add; one workgroup then averages sigma over the units of every tile
// and fires the tiles whose mean lies in the lowest q fraction of the layer's
// tiles, and those tiles' rows take their extra blocks into the CSR.
// Each branch is reduced to a threshold key T (the rank-k key, found by bisection
// on the order-preserving integer image of the fp32 value) plus a count of
// threshold ties admitted in index order.  All sums use a fixed reduction tree, so
// a row's result is reproducible run to run.
//
// CSR: a single-workgroup exclusive scan of the row counts, then one wave per row
// writes the set bits of its mask in ascending order.
#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"
#include "slot_bits.h"

namespace bsa {

namespace {

// ------------------------------------------------------------------ scores

// One workgroup of four waves per 128 x 128 tile of the causal lower triangle;
// wave w computes the 64 x 64 sub-tile (w / 2, w % 2) as 2 x 2 products of 32 x 32,
// so every operand read from LDS feeds two products.  The products run on the
// bf16 matrix cores (V_MFMA_F32_32X32X16_BF16) with each fp32 centroid split into
// a bf16 head and a bf16 remainder, x = hi + lo with |x - hi - lo| <= 2^-18 |x|,
// and three products per step, hi*hi + hi*lo + lo*hi (the dropped lo*lo is below
// 2^-18 of |q_d k_d|), accumulated in fp32: every score is within about 3e-6 of
// ||qbar|| ||kbar|| of the exact one, at three sixteenths of the fp32 matrix-core
// cost.  The tile's 128 query and 128 key centroids are staged through LDS 32
// dimensions at a time with coalesced 16-byte loads (the next 32 loaded into
// registers while the current ones are multiplied), split as they are stored;
// a staged row holds its 32 heads then its 32 remainders and is padded to 144
// bytes (9 x 16), so the 16-byte operand reads of 16 consecutive rows fall on 16
// different 16-byte bank groups.  The grid enumerates the lower-triangle tiles
// only (tile t of row it = the largest with it(it+1)/2 <= t), so consecutive
// workgroups, which the dispatcher deals round-robin to the eight XCDs, spread
// the work evenly; a square grid with the upper tiles exiting would give XCD k
// only the tile rows it = k (mod 8).
__device__ __forceinline__ void split_bf16x4(const f32x4& x, u32x2& hi, u32x2& lo) {
  hi = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  const float r0 = x[0] - __uint_as_float(hi[0] << 16);
  const float r1 = x[1] - __uint_as_float(hi[0] & 0xFFFF0000u);
  const float r2 = x[2] - __uint_as_float(hi[1] << 16);
  const float r3 = x[3] - __uint_as_float(hi[1] & 0xFFFF0000u);
  lo = u32x2{pack_bf16x2(r0, r1), pack_bf16x2(r2, r3)};
}

constexpr int kScoreRow = 144;  // bytes per staged row: 32 bf16 heads, 32 remainders, pad

__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qc,
                                                    const float* __restrict__ kc,
                                                    float* __restrict__ scores, int nb, int D,
                                                    int G, int per_group) {
  const int t = blockIdx.x, u = blockIdx.y;
  int it = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((it + 1) * (it + 2) / 2 <= t) ++it;  // float rounding, either way
  while (it * (it + 1) / 2 > t) --it;
  const int jt = t - it * (it + 1) / 2;
  __shared__ __attribute__((aligned(16))) unsigned char As[128 * kScoreRow], Bs[128 * kScoreRow];
  const int tid = threadIdx.x, l = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = w >> 1, wj = w & 1, hf = l >> 5;
  const int g = per_group ? u : u / G;
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{0};
  f32x4 av[4], bv[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int idx = tid + 256 * t4, row = idx >> 3, c4 = (idx & 7) * 4;
      const int ia = min(it * 128 + row, nb - 1), jb = min(jt * 128 + row, nb - 1);
      av[t4] = *(const f32x4*)(qc + ((size_t)u * nb + ia) * D + k0 + c4);
      bv[t4] = *(const f32x4*)(kc + ((size_t)g * nb + jb) * D + k0 + c4);
    }
  };
  load(0);
  for (int k0 = 0; k0 < D; k0 += 32) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int idx = tid + 256 * t4, row = idx >> 3, c4 = (idx & 7) * 4;
      u32x2 h, r;
      split_bf16x4(av[t4], h, r);
      *(u32x2*)(As + row * kScoreRow + c4 * 2) = h;
      *(u32x2*)(As + row * kScoreRow + 64 + c4 * 2) = r;
      split_bf16x4(bv[t4], h, r);
      *(u32x2*)(Bs + row * kScoreRow + c4 * 2) = h;
      *(u32x2*)(Bs + row * kScoreRow + 64 + c4 * 2) = r;
    }
    __syncthreads();
    if (k0 + 32 < D) load(k0 + 32);
    // A: query rows wi*64 + 32x + l%32, B: key rows wj*64 + 32y + l%32; lane half
    // hf takes dimensions 8hf..8hf+7 of each 16-dimension step s
    const unsigned char* ar = As + (wi * 64 + (l & 31)) * kScoreRow + hf * 16;
    const unsigned char* br = Bs + (wj * 64 + (l & 31)) * kScoreRow + hf * 16;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        ah[x] = *(const bf16x8*)(ar + x * 32 * kScoreRow + s * 32);
        al[x] = *(const bf16x8*)(ar + x * 32 * kScoreRow + 64 + s * 32);
        bh[x] = *(const bf16x8*)(br + x * 32 * kScoreRow + s * 32);
        bl[x] = *(const bf16x8*)(br + x * 32 * kScoreRow + 64 + s * 32);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[x], bl[y], acc[x][y], 0, 0, 0);
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[x], bh[y], acc[x][y], 0, 0, 0);
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[x], bh[y], acc[x][y], 0, 0, 0);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int j = jt * 128 + wj * 64 + y * 32 + (l & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = it * 128 + wi * 64 + x * 32 + (v >> 2) * 8 + hf * 4 + (v & 3);
        if (i < nb && j <= i) scores[((size_t)u * nb + i) * nb + j] = acc[x][y][v];
      }
    }
}

// ------------------------------------------------------------------ selection

struct SelArgs {
  const float* scores;
  const float* qn;
  const float* kr;
  float* bound_out;
  uint8_t* gate_out;
  unsigned long long* mask;
  int* counts;
  int nb, nw, rows, G, per_group;
  int units, i0, ni;  // register form: this launch's query blocks [i0, i0 + ni) of every unit
  int top_k, force_sink, gate, gate_factor;
  float gate_threshold, tau_log2e, mass_threshold;
  double rescue_fraction;
  int use_b, use_p, per_wave_floats;
  // sigma gate (gate == 2): per-row cut margin, the blocks that top-(rho*k) adds
  // beyond the row's kept set, and their count
  float* sigma;
  unsigned long long* mask_x;
  int* counts_x;
  // set to 1 when some row's kept set does not fit the output (cleared here,
  // written by the scan or, for the padded list, by compaction)
  int* overflow;
};

// Clears the overflow word once per launch (every launch of a selection comes
// before its compaction on the stream).
__device__ __forceinline__ void clear_overflow(const SelArgs& a) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.overflow = 0;
}

__device__ __forceinline__ bool is_cand(int j, int i, int sink) {
  return j < i && !(sink && j == 0);
}

// inverse of float_key
__device__ __forceinline__ float key_float(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ unsigned wave_max_u(unsigned x) { return wave_max_uint(x); }

__device__ __forceinline__ unsigned wave_min_u(unsigned x) { return wave_min_uint(x); }

// Cut margin of a top-k decision from the keys of s(0) (best candidate), s(k-1)
// (last kept) and s(k) (first dropped): (s(k-1) - s(k)) / (s(0) - s(k)), and 0
// when s(0) = s(k) (every score down to the cut tied).
__device__ __forceinline__ float cut_margin(unsigned k0, unsigned klast, unsigned kdrop) {
  const float s0 = key_float(k0), a = key_float(klast), b = key_float(kdrop);
  return s0 == b ? 0.f : (a - b) / (s0 - b);
}

// number of candidates whose key(vals[j]) >= X
__device__ int count_ge(const float* vals, int nslots, int i, int sink, unsigned X) {
  const int l = lane_id();
  int c = 0;
  for (int e = 0; e < nslots; ++e) {
    const int j = e * 64 + l;
    c += (is_cand(j, i, sink) && float_key(vals[j]) >= X) ? 1 : 0;
  }
  return wave_sum_int(c);
}

// Threshold of the top-k over candidates: (T, need) such that the kept set is
// {key > T} plus the first `need` candidates with key == T in index order.
__device__ void topk_threshold(const float* vals, int nslots, int i, int sink, int nc, int k,
                               unsigned& T, int& need) {
  if (k >= nc) {  // every candidate
    T = 0u;
    need = nc;
    return;
  }
  if (k <= 0) {
    T = 0xFFFFFFFFu;
    need = 0;
    return;
  }
  // Bisection for the largest key t with at least k candidates >= t.  A probe x
  // with exactly k candidates >= x already decides the kept set ({key >= x},
  // the same k candidates the full bisection keeps), so the search stops there.
  unsigned t = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned x = t | (1u << bit);
    const int c = count_ge(vals, nslots, i, sink, x);
    if (c >= k) t = x;
    if (c == k) break;
  }
  const int gt = (t == 0xFFFFFFFFu) ? 0 : count_ge(vals, nslots, i, sink, t + 1u);
  T = t;
  need = k - gt;
}

// mass of candidates with key(s) >= X (fixed-order sum)
__device__ float mass_ge(const float* s, const float* p, int nslots, int i, int sink, unsigned X) {
  const int l = lane_id();
  float m = 0.f;
  for (int e = 0; e < nslots; ++e) {
    const int j = e * 64 + l;
    if (is_cand(j, i, sink) && float_key(s[j]) >= X) m += p[j];
  }
  return wave_sum(m);
}

__global__ __launch_bounds__(256) void select_kernel(SelArgs a) {
  extern __shared__ float sm[];
  clear_overflow(a);
  const int l = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * (blockDim.x >> 6) + wave;
  if (w >= a.rows) return;  // no workgroup barriers below
  const int nb = a.nb;
  // longest rows first: wave w takes query block nb - 1 - w / U of unit w % U, so
  // the last workgroups dispatched hold the shortest rows
  const int U = a.rows / nb;
  const int u = w % U, i = nb - 1 - w / U;
  const int row = u * nb + i;
  const int g = a.per_group ? u : u / a.G;
  float* s = sm + (size_t)wave * a.per_wave_floats;
  float* b = s + a.nw * 64;
  float* p = b + (a.use_b ? a.nw * 64 : 0);
  const int nslots = i / 64 + 1;
  const int sink = a.force_sink;
  const int nc = i > 0 ? i - (sink ? 1 : 0) : 0;
  const float* srow = a.scores + ((size_t)u * nb + i) * nb;
  const float qnv = a.use_b ? a.qn[(size_t)u * nb + i] : 0.f;
  for (int e = 0; e < nslots; ++e) {
    const int j = e * 64 + l;
    if (j <= i) {
      const float sv = srow[j];
      s[j] = sv;
      if (a.use_b) {
        const float bv = fmaf(qnv, a.kr[(size_t)g * nb + j], sv);
        b[j] = bv;
        if (a.bound_out) a.bound_out[((size_t)u * nb + i) * nb + j] = bv;
      }
    }
  }
  // (each lane reads back only the entries it wrote, so no barrier is needed)

  // softmax statistics over the candidates (gate and mass)
  float s0 = -INFINITY, zsum = 0.f;
  const bool need_soft = (a.gate == 1 && a.top_k > 0) || a.use_p;
  const bool sig = a.gate == 2 && a.top_k > 0;
  if (need_soft && nc > 0) {
    float mx = -INFINITY;
    for (int e = 0; e < nslots; ++e) {
      const int j = e * 64 + l;
      if (is_cand(j, i, sink)) mx = fmaxf(mx, s[j]);
    }
    s0 = wave_max(mx);
    float z = 0.f;
    for (int e = 0; e < nslots; ++e) {
      const int j = e * 64 + l;
      if (is_cand(j, i, sink)) {
        const float w = exp2f((s[j] - s0) * a.tau_log2e);
        z += w;
        if (a.use_p) p[j] = w;
      }
    }
    zsum = wave_sum(z);
    if (a.use_p) {
      const float inv = 1.0f / zsum;
      for (int e = 0; e < nslots; ++e) {
        const int j = e * 64 + l;
        if (is_cand(j, i, sink)) p[j] *= inv;
      }
    }
  }

  // top-k branch (with the optional gate)
  unsigned Tk = 0xFFFFFFFFu;
  int needk = 0;
  bool fired = false;
  if (a.top_k > 0) {
    if (a.gate == 1 && nc >= 2) {
      // runner-up: best candidate other than the first (lowest-index) maximum
      int jmax = 0x7FFFFFFF;
      for (int e = 0; e < nslots; ++e) {
        const int j = e * 64 + l;
        if (is_cand(j, i, sink) && s[j] == s0) jmax = min(jmax, j);
      }
      jmax = wave_min_int(jmax);
      float m2 = -INFINITY;
      for (int e = 0; e < nslots; ++e) {
        const int j = e * 64 + l;
        if (is_cand(j, i, sink) && j != jmax) m2 = fmaxf(m2, s[j]);
      }
      const float s1 = wave_max(m2);
      const float gap = (1.0f - exp2f((s1 - s0) * a.tau_log2e)) / zsum;
      fired = gap < a.gate_threshold;
    }
    const int keff = a.top_k * (fired ? a.gate_factor : 1);
    topk_threshold(s, nslots, i, sink, nc, keff, Tk, needk);
  }
  // sigma gate: the threshold of the expanded budget rho*k
  unsigned Tx = 0xFFFFFFFFu;
  int needx = 0;
  if (sig) topk_threshold(s, nslots, i, sink, nc, a.top_k * a.gate_factor, Tx, needx);

  // base branch: shortest prefix of the order reaching mass mu
  unsigned Tm = 0xFFFFFFFFu;
  int needm = 0;
  if (a.use_p && nc > 0) {
    unsigned t = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned x = t | (1u << bit);
      if (mass_ge(s, p, nslots, i, sink, x) >= a.mass_threshold) t = x;
    }
    if (mass_ge(s, p, nslots, i, sink, t) < a.mass_threshold) {
      Tm = 0u;  // the total falls short in float32: keep every candidate
      needm = nc;
    } else {
      Tm = t;
      float cum = (t == 0xFFFFFFFFu) ? 0.f : mass_ge(s, p, nslots, i, sink, t + 1u);
      // admit ties at T in index order until the mass is reached
      for (int e = 0; e < nslots && cum < a.mass_threshold; ++e) {
        const int j = e * 64 + l;
        unsigned long long tie = ballot64(is_cand(j, i, sink) && float_key(s[j]) == t);
        while (tie && cum < a.mass_threshold) {
          const int src = __builtin_ctzll(tie);
          cum += __shfl(p[e * 64 + l], src);
          ++needm;
          tie &= tie - 1;
        }
      }
    }
  }

  // rescue branch: top ceil(phi*|C_i|) by the bound
  unsigned Tr = 0xFFFFFFFFu;
  int needr = 0;
  if (a.use_b && nc > 0) {
    int nr = (int)ceil(a.rescue_fraction * (double)nc);
    nr = nr < nc ? nr : nc;
    topk_threshold(b, nslots, i, sink, nc, nr, Tr, needr);
  }

  // union and mask emission (with the sigma gate: the cut statistics of the
  // top-k set and the expansion bits, blocks of top-(rho*k) not kept otherwise)
  int runk = 0, runm = 0, runr = 0, runx = 0, count = 0, countx = 0;
  unsigned ktop = 0u, kin = 0xFFFFFFFFu, kout = 0u;
  const unsigned long long lt = lanemask_lt();
  unsigned long long* mrow = a.mask + (size_t)row * a.nw;
  for (int e = 0; e < nslots; ++e) {
    const int j = e * 64 + l;
    const bool c = is_cand(j, i, sink);
    bool keep = (j == i) || (sink && j == 0 && j <= i);
    bool inx = false;
    if (a.top_k > 0) {
      const unsigned key = c ? float_key(s[j]) : 0u;
      const unsigned long long tie = ballot64(c && key == Tk);
      const bool ink = c && (key > Tk || ((tie >> l) & 1ull && runk + __popcll(tie & lt) < needk));
      keep |= ink;
      runk += __popcll(tie);
      if (sig) {
        if (c) ktop = max(ktop, key);
        if (ink) kin = min(kin, key);
        else if (c) kout = max(kout, key);
        const unsigned long long tx = ballot64(c && key == Tx);
        inx = c && (key > Tx || ((tx >> l) & 1ull && runx + __popcll(tx & lt) < needx));
        runx += __popcll(tx);
      }
    }
    if (a.use_p) {
      const unsigned key = c ? float_key(s[j]) : 0u;
      const unsigned long long tie = ballot64(c && key == Tm);
      keep |= c && (key > Tm || ((tie >> l) & 1ull && runm + __popcll(tie & lt) < needm));
      runm += __popcll(tie);
    }
    if (a.use_b) {
      const unsigned key = c ? float_key(b[j]) : 0u;
      const unsigned long long tie = ballot64(c && key == Tr);
      keep |= c && (key > Tr || ((tie >> l) & 1ull && runr + __popcll(tie & lt) < needr));
      runr += __popcll(tie);
    }
    const unsigned long long word = ballot64(keep && j <= i);
    if (l == 0) mrow[e] = word;
    count += __popcll(word);
    if (sig) {
      const unsigned long long wx = ballot64(inx && !keep);
      if (l == 0) a.mask_x[(size_t)row * a.nw + e] = wx;
      countx += __popcll(wx);
    }
  }
  if (sig) {
    ktop = wave_max_u(ktop);
    kin = wave_min_u(kin);
    kout = wave_max_u(kout);
  }
  if (l == 0) {
    a.counts[row] = count;
    if (sig) {
      a.counts_x[row] = countx;
      a.sigma[row] = nc > a.top_k ? cut_margin(ktop, kin, kout) : 0.f;
    } else if (a.gate_out) {
      a.gate_out[row] = fired ? 1 : 0;
    }
  }
}

// ------------------------------------------------------------------ selection, register form
// Rows of up to 64*SPL blocks keep their order-preserving keys in registers
// (slot e of lane l holds block j = 64e + l).  A threshold probe is then one
// compare per slot plus a ballot popcount (scalar), with no LDS traffic and no
// cross-lane reduction; the base branch extracts maxima one at a time in the
// ranking order (the usual case needs a handful) and falls back to bisection
// on fixed-tree mass sums when more than 16 blocks are needed.

template <int SPL>
struct RowKeys {
  static_assert(SPL >= 1 && SPL <= 128, "register form: at most 128 slots per lane");
  unsigned k[SPL];
  SlotBits<SPL> cand_bits;  // bit e: slot e of this lane is a candidate
  __device__ __forceinline__ bool cand(int e) const { return cand_bits.get(e); }
};

// number of candidates with key >= x (wave-uniform).  Slots that hold no
// candidate keep key 0, below every probe (x >= 1), so no candidacy test is needed.
// Slots past the row (e >= nsl) hold key 0 as well, so the row is counted in
// chunks of 8 slots behind one uniform branch each.  The widest forms (64 and 128
// slots, few waves per SIMD) count per lane on the VALU and sum the lanes once;
// the others take a ballot popcount per slot on the scalar unit.
template <int SPL>
__device__ __forceinline__ int count_ge_reg(const RowKeys<SPL>& r, int nsl, unsigned x) {
  constexpr int CH = SPL < 8 ? SPL : 8;
  int c = 0;
#pragma unroll
  for (int e0 = 0; e0 < SPL; e0 += CH)
    if (e0 < nsl) {
#pragma unroll
      for (int e = e0; e < e0 + CH; ++e) {
        if constexpr (SPL >= 64)
          c += r.k[e] >= x ? 1 : 0;
        else
          c += __popcll(ballot64(r.k[e] >= x));
      }
    }
  if constexpr (SPL >= 64) c = wave_sum_int(c);
  return c;
}

template <int SPL>
__device__ void topk_reg(const RowKeys<SPL>& r, int nsl, int nc, int k, unsigned& T, int& need) {
  if (k >= nc) {
    T = 0u;
    need = nc;
    return;
  }
  if (k <= 0) {
    T = 0xFFFFFFFFu;
    need = 0;
    return;
  }
  // Bisection for the largest key t with at least k candidates >= t (early exit
  // as in topk_threshold: exactly k candidates >= x decide the set).  For k <= 64
  // it starts below the bits that the k-th largest lane maximum m and the largest
  // key share: t lies in [m, max] (k lanes hold a key >= m), so the full bisection
  // would set exactly those bits (probes at or below m count >= k, above max count
  // 0) and only then reach the bits where m and max differ.  The lane maxima are
  // ranked by ballots, which cost a compare and a popcount per probe instead of a
  // pass over every slot.
  unsigned t = 0u;
  int top = 31;
  if (k <= 64) {
    unsigned lm = 0u;  // non-candidate slots hold key 0
#pragma unroll
    for (int e = 0; e < SPL; ++e)
      if (e < nsl) lm = max(lm, r.k[e]);
    unsigned m = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned x = m | (1u << bit);
      if (__popcll(ballot64(lm >= x)) >= k) m = x;
    }
    const unsigned kmax = wave_max_uint(lm);
    const unsigned diff = m ^ kmax;
    top = diff ? 31 - __builtin_clz(diff) : -1;
    t = top < 0 ? m : (top == 31 ? 0u : (m & ~((2u << top) - 1u)));
  }
  for (int bit = top; bit >= 0; --bit) {
    const unsigned x = t | (1u << bit);
    const int c = count_ge_reg(r, nsl, x);
    if (c >= k) t = x;
    if (c == k) break;
  }
  need = k - (t == 0xFFFFFFFFu ? 0 : count_ge_reg(r, nsl, t + 1u));
  T = t;
}

// FULL = false compiles the top-k and gate branches only (the rescue keys and the
// mass probabilities would not fit in registers at 128 slots).  SIG compiles the
// sigma gate's per-row part (its extra state stays out of the other forms).
// (the widest forms are held to the registers of two waves per SIMD, the 32-slot
// form with every branch to three, the 64-slot top-k-only one to four and the
// 16-slot one to five: a wave with its SIMD to itself waits out every load and
// reduction latency of its row, and a few spilled registers cost less; at 16 slots
// the fifth wave takes 9 % off the selection of 128K-token layers, at 64 the
// fourth 2 % off that of 1M-token layers)
template <int SPL, bool FULL, bool SIG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    (SPL >= 128 || (SPL == 64 && FULL && !SIG)) ? 2
    : (SPL == 32 && FULL)                        ? 3
    : (SPL == 64 && !FULL)                       ? 4
    : (SPL == 16 && FULL)                        ? 5
                                                 : 1)))
void select_reg_kernel(SelArgs a) {
  clear_overflow(a);
  const bool use_b = FULL && a.use_b, use_p = FULL && a.use_p;
  const int l = lane_id();
  // (the wave index through readfirstlane: row, i and the slot count are then
  // known to be wave-uniform, and the per-slot conditions below scalar branches)
  const int r = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = a.nb;
  if (r >= a.units * a.ni) return;  // no workgroup barriers below
  // longest rows first: query block i0 + ni - 1 - r / units of unit r % units, so
  // the last workgroups dispatched hold the shortest rows
  const int u = r % a.units, i = a.i0 + a.ni - 1 - r / a.units;
  const int row = u * nb + i;
  const int g = a.per_group ? u : u / a.G;
  const int sink = a.force_sink;
  const int nc = i > 0 ? i - (sink ? 1 : 0) : 0;
  const int nsl = i / 64 + 1;
  const float* srow = a.scores + ((size_t)u * nb + i) * nb;
  const float qnv = use_b ? a.qn[(size_t)u * nb + i] : 0.f;

  RowKeys<SPL> sr, br;
  sr.cand_bits.clear();
  // the row is read in chunks of up to 32 slots per lane, each chunk's loads issued
  // together (indices clamped into the row, one wait per chunk) rather than one
  // load and one wait per slot
  // (32 slots per chunk for the 32- and 64-slot top-k-only forms, 16 for the
  // 128-slot one, whose 256 registers leave no room for more, the whole row up to
  // 16 slots but 8 for the other forms with every branch)
  constexpr int CH = FULL ? (SPL <= 8 ? SPL : 8)
                          : (SPL <= 16 ? SPL : SPL >= 128 ? 16 : SPL > 32 ? 32 : SPL);
#pragma unroll
  for (int e0 = 0; e0 < SPL; e0 += CH) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      sr.k[e0 + c] = 0u;
      br.k[e0 + c] = 0u;
    }
    if (e0 < nsl) {
      float sv[CH], kv[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int j = min((e0 + c) * 64 + l, i);
        sv[c] = srow[j];
        if (use_b) kv[c] = a.kr[(size_t)g * nb + j];
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int e = e0 + c, j = e * 64 + l;
        if (e < nsl && j <= i) {
          sr.k[e] = float_key(sv[c]);
          if (use_b) {
            const float bv = fmaf(qnv, kv[c], sv[c]);
            br.k[e] = float_key(bv);
            if (a.bound_out) a.bound_out[((size_t)u * nb + i) * nb + j] = bv;
          }
          if (is_cand(j, i, sink)) {
            sr.cand_bits.set(e);
          } else {
            sr.k[e] = 0u;  // forced blocks are no candidates: below every probe
            br.k[e] = 0u;
          }
        }
      }
    }
  }
  br.cand_bits = sr.cand_bits;

  // softmax statistics over the candidates (gate and mass)
  float s0 = -INFINITY, zsum = 0.f;
  unsigned kmax = 0u;
  const bool need_soft = (a.gate == 1 && a.top_k > 0) || use_p;
  const bool sig = SIG && a.gate == 2 && a.top_k > 0;
  if (need_soft && nc > 0) {
    unsigned km = 0u;
#pragma unroll
    for (int e = 0; e < SPL; ++e)
      if (e < nsl && sr.cand(e)) km = max(km, sr.k[e]);
    km = wave_max_uint(km);
    kmax = km;
    s0 = key_float(kmax);
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < SPL; ++e)
      if (e < nsl && sr.cand(e)) z += exp2f((key_float(sr.k[e]) - s0) * a.tau_log2e);
    zsum = wave_sum(z);
  }

  // top-k branch (with the optional gate)
  unsigned Tk = 0xFFFFFFFFu;
  int needk = 0;
  bool fired = false;
  if (a.top_k > 0) {
    if (a.gate == 1 && nc >= 2) {
      int jm = 0x7FFFFFFF;
#pragma unroll
      for (int e = SPL - 1; e >= 0; --e)
        if (e < nsl && sr.cand(e) && sr.k[e] == kmax) jm = e * 64 + l;
      jm = wave_min_int(jm);
      unsigned k2 = 0u;
#pragma unroll
      for (int e = 0; e < SPL; ++e)
        if (e < nsl && sr.cand(e) && e * 64 + l != jm) k2 = max(k2, sr.k[e]);
      k2 = wave_max_uint(k2);
      const float gap = (1.0f - exp2f((key_float(k2) - s0) * a.tau_log2e)) / zsum;
      fired = gap < a.gate_threshold;
    }
    topk_reg(sr, nsl, nc, a.top_k * (fired ? a.gate_factor : 1), Tk, needk);
  }
  // sigma gate: the threshold of the expanded budget rho*k
  unsigned Tx = 0xFFFFFFFFu;
  int needx = 0;
  if (sig) topk_reg(sr, nsl, nc, a.top_k * a.gate_factor, Tx, needx);

  // base branch: shortest prefix of the ranking whose mass reaches mu
  SlotBits<SPL> taken;  // extraction result (bits per slot of this lane)
  taken.clear();
  bool by_extraction = true;
  unsigned Tm = 0xFFFFFFFFu;
  int needm = 0;
  if (use_p && nc > 0) {
    float cum = 0.f;
    int steps = 0;
    bool done = false;
    while (!done && steps < 16) {
      unsigned bk = 0u;
      int bj = 0x7FFFFFFF;
#pragma unroll
      for (int e = 0; e < SPL; ++e)
        if (e < nsl && sr.cand(e) && !taken.get(e) && sr.k[e] > bk) {
          bk = sr.k[e];
          bj = e * 64 + l;
        }
      // the largest key, then the lowest block index holding it (each lane's bj is
      // its lowest slot with its own largest key)
      const unsigned kb = wave_max_uint(bk);
      bj = wave_min_int(bk == kb ? bj : 0x7FFFFFFF);
      bk = kb;
      if (bj == 0x7FFFFFFF) break;  // every candidate taken
      cum += exp2f((key_float(bk) - s0) * a.tau_log2e) / zsum;
      if ((bj & 63) == l) taken.set(bj >> 6);
      ++steps;
      done = cum >= a.mass_threshold;
    }
    if (!done && steps >= 16) {
      // many blocks needed: bisection on the mass of {key >= x} (fixed-tree sums)
      by_extraction = false;
      float pe[SPL];  // each candidate's probability, computed once for all steps
#pragma unroll
      for (int e = 0; e < SPL; ++e)
        pe[e] = (e < nsl && sr.cand(e)) ? exp2f((key_float(sr.k[e]) - s0) * a.tau_log2e) / zsum
                                        : 0.f;
      auto mass_ge = [&](unsigned x) {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < SPL; ++e)
          if (e < nsl && sr.cand(e) && sr.k[e] >= x) m += pe[e];
        return wave_sum(m);
      };
      unsigned t = 0u;
      for (int bit = 31; bit >= 0; --bit) {
        const unsigned x = t | (1u << bit);
        if (mass_ge(x) >= a.mass_threshold) t = x;
      }
      if (mass_ge(t) < a.mass_threshold) {
        Tm = 0u;
        needm = nc;
      } else {
        Tm = t;
        float c2 = (t == 0xFFFFFFFFu) ? 0.f : mass_ge(t + 1u);
#pragma unroll
        for (int e = 0; e < SPL; ++e) {
          if (e >= nsl || c2 >= a.mass_threshold) continue;
          unsigned long long tie = ballot64(sr.cand(e) && sr.k[e] == t);
          while (tie && c2 < a.mass_threshold) {
            const int src = __builtin_ctzll(tie);
            c2 += exp2f((key_float(t) - s0) * a.tau_log2e) / zsum;
            ++needm;
            tie &= tie - 1;
            (void)src;
          }
        }
      }
    }
  }

  // rescue branch: top ceil(phi*|C_i|) by the bound
  unsigned Tr = 0xFFFFFFFFu;
  int needr = 0;
  if (use_b && nc > 0) {
    int nr = (int)ceil(a.rescue_fraction * (double)nc);
    nr = nr < nc ? nr : nc;
    topk_reg(br, nsl, nc, nr, Tr, needr);
  }

  // union and mask emission (with the sigma gate: the cut statistics of the
  // top-k set and the expansion bits, blocks of top-(rho*k) not kept otherwise)
  int runk = 0, runm = 0, runr = 0, runx = 0, count = 0, countx = 0;
  unsigned ktop = 0u, kin = 0xFFFFFFFFu, kout = 0u;
  const unsigned long long lt = lanemask_lt();
  unsigned long long* mrow = a.mask + (size_t)row * a.nw;
#pragma unroll
  for (int e = 0; e < SPL; ++e) {
    if (e >= nsl) continue;
    const int j = e * 64 + l;
    const bool c = sr.cand(e);
    bool keep = (j == i) || (sink && j == 0 && j <= i);
    bool inx = false;
    if (a.top_k > 0) {
      const unsigned long long tie = ballot64(c && sr.k[e] == Tk);
      const bool ink =
          c && (sr.k[e] > Tk || ((tie >> l) & 1ull && runk + __popcll(tie & lt) < needk));
      keep |= ink;
      runk += __popcll(tie);
      if (sig) {
        if (c) ktop = max(ktop, sr.k[e]);
        if (ink) kin = min(kin, sr.k[e]);
        else if (c) kout = max(kout, sr.k[e]);
        const unsigned long long tx = ballot64(c && sr.k[e] == Tx);
        inx = c && (sr.k[e] > Tx || ((tx >> l) & 1ull && runx + __popcll(tx & lt) < needx));
        runx += __popcll(tx);
      }
    }
    if (use_p) {
      if (by_extraction) {
        keep |= taken.get(e);
      } else {
        const unsigned long long tie = ballot64(c && sr.k[e] == Tm);
        keep |= c && (sr.k[e] > Tm || ((tie >> l) & 1ull && runm + __popcll(tie & lt) < needm));
        runm += __popcll(tie);
      }
    }
    if (use_b) {
      const unsigned long long tie = ballot64(c && br.k[e] == Tr);
      keep |= c && (br.k[e] > Tr || ((tie >> l) & 1ull && runr + __popcll(tie & lt) < needr));
      runr += __popcll(tie);
    }
    const unsigned long long word = ballot64(keep && j <= i);
    if (l == 0) mrow[e] = word;
    count += __popcll(word);
    if (sig) {
      const unsigned long long wx = ballot64(inx && !keep);
      if (l == 0) a.mask_x[(size_t)row * a.nw + e] = wx;
      countx += __popcll(wx);
    }
  }
  if (sig) {
    ktop = wave_max_u(ktop);
    kin = wave_min_u(kin);
    kout = wave_max_u(kout);
  }
  if (l == 0) {
    a.counts[row] = count;
    if (sig) {
      a.counts_x[row] = countx;
      a.sigma[row] = nc > a.top_k ? cut_margin(ktop, kin, kout) : 0.f;
    } else if (a.gate_out) {
      a.gate_out[row] = fired ? 1 : 0;
    }
  }
}

// ------------------------------------------------------------------ sigma gate, per tile
// One workgroup for the layer.  Tile i has a cut when |C_i| > k; its signal is
// the mean of sigma over the U units (summed in unit order).  With T tiles that
// have a cut and r = floor(q*T) (in double), tile i fires when at most r of
// them have a mean <= its own, i.e. when its mean lies strictly below the
// (r+1)-th smallest, found by bisection on the order-preserving keys.  The
// per-tile decision is left in fire[]: a row-parallel pass adds the expansion
// counts of fired rows before the scan, and the compaction their bits.
constexpr unsigned kNoCut = 0xFFFFFFFFu;  // key of a tile without a cut (never a mean's key)

__global__ __launch_bounds__(1024) void sigma_tile_kernel(const float* __restrict__ sigma,
                                                          unsigned* __restrict__ gkeys,
                                                          uint8_t* __restrict__ fire, int U,
                                                          int nb, int k, int sink, float q,
                                                          int keys_in_lds) {
  extern __shared__ unsigned skeys[];
  __shared__ int part[2][16];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  unsigned* keys = keys_in_lds ? skeys : gkeys;
  int parity = 0;
  // one barrier per sum: consecutive sums alternate between the two halves of
  // part[], and a half is rewritten only after the barrier of the sum in between
  auto block_sum = [&](int v) {
    v = wave_sum_int(v);
    if (l == 0) part[parity][w] = v;
    __syncthreads();
    int tot = 0;
    for (int x = 0; x < 16; ++x) tot += part[parity][x];
    parity ^= 1;
    return tot;
  };
  int mine = 0;
  for (int i = t; i < nb; i += 1024) {
    const int nc = i > 0 ? i - sink : 0;
    unsigned key = kNoCut;
    if (nc > k) {
      float sum = 0.f;
      int u = 0;
      for (; u + 8 <= U; u += 8) {  // eight loads in flight, added in unit order
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = sigma[(size_t)(u + e) * nb + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += v[e];
      }
      for (; u < U; ++u) sum += sigma[(size_t)u * nb + i];
      key = float_key(sum / (float)U);
      ++mine;
    }
    keys[i] = key;
  }
  const int T = block_sum(mine);  // (its barrier also publishes keys[])
  const int r = (int)floor((double)q * (double)T);
  const int need = T - r;  // keys at or above the (r+1)-th smallest
  unsigned tq = 0xFFFFFFFFu;  // r >= T: every tile with a cut fires
  if (need > 0) {
    tq = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned x = tq | (1u << bit);
      int c = 0;
      for (int i = t; i < nb; i += 1024) c += (keys[i] != kNoCut && keys[i] >= x) ? 1 : 0;
      if (block_sum(c) >= need) tq = x;
    }
  }
  for (int i = t; i < nb; i += 1024) fire[i] = (keys[i] != kNoCut && keys[i] < tq) ? 1 : 0;
}

// ------------------------------------------------------------------ CSR
//
// Row offsets in three steps: the kept counts are summed per run of 64 rows (one
// wave per run), one workgroup scans the run sums, and the compaction, one wave
// per row, adds the counts of the rows before it in its run (one coalesced load
// and a wave sum) to its run's offset.

__global__ __launch_bounds__(256) void run_sum_kernel(const int* __restrict__ counts,
                                                      int* __restrict__ run_sum, int rows) {
  const int l = lane_id();
  const int run = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (run * 64 >= rows) return;
  const int r = run * 64 + l;
  const int c = wave_sum_int(r < rows ? counts[r] : 0);
  if (l == 0) run_sum[run] = c;
}

// Exclusive scan of the run sums (`rows` values here) in one workgroup: thread t
// owns a contiguous chunk (a multiple of 4 values, read and written as 16-byte
// vectors), the chunk sums are scanned with wave shuffles and one LDS step across
// the 16 waves; the total goes to row_ptr[rows].  Offsets are clamped to the
// col_idx capacity, so a reader of the CSR can never index past the buffer; the
// capacity bound makes the clamp a no-op, and a total past it (kept sets larger
// than the parameters allow) sets the overflow word.
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ counts,
                                                    int32_t* __restrict__ row_ptr, int rows,
                                                    int64_t capacity, int* __restrict__ overflow) {
  __shared__ int wsum[16];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int chunk = (((rows + 1023) / 1024) + 3) & ~3;
  const int r0 = min(rows, t * chunk), r1 = min(rows, r0 + chunk);
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  int sum = 0;
  for (int r = r0; r < r1; r += 4) {
    if (r + 4 <= r1) {
      const i32x4 v = *(const i32x4*)(counts + r);
      sum += v[0] + v[1] + v[2] + v[3];
    } else {
      for (int q = r; q < r1; ++q) sum += counts[q];
    }
  }
  int x = sum;  // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(x, o);
    if (l >= o) x += v;
  }
  if (l == 63) wsum[w] = x;
  __syncthreads();
  int before = 0;
  for (int ww = 0; ww < w; ++ww) before += wsum[ww];
  int64_t run = (int64_t)before + x - sum;  // exclusive prefix of this chunk
  auto clampc = [&](int64_t v) { return (int32_t)(v < capacity ? v : capacity); };
  for (int r = r0; r < r1; r += 4) {
    if (r + 4 <= r1) {
      const i32x4 v = *(const i32x4*)(counts + r);
      i32x4 o;
      o[0] = clampc(run);
      o[1] = clampc(run + v[0]);
      o[2] = clampc(run + v[0] + v[1]);
      o[3] = clampc(run + v[0] + v[1] + v[2]);
      *(i32x4*)(row_ptr + r) = o;
      run += v[0] + v[1] + v[2] + v[3];
    } else {
      for (int q = r; q < r1; ++q) {
        row_ptr[q] = clampc(run);
        run += counts[q];
      }
    }
  }
  if (t == 1023) {
    row_ptr[rows] = clampc((int64_t)before + x);
    *overflow = (int64_t)before + x > capacity ? 1 : 0;
  }
}

// Sigma gate: a row whose tile fired also keeps its expansion blocks.
__global__ __launch_bounds__(256) void expand_counts_kernel(int* __restrict__ counts,
                                                            const int* __restrict__ counts_x,
                                                            const uint8_t* __restrict__ fire,
                                                            int rows, int nb) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row < rows && fire[row % nb]) counts[row] += counts_x[row];
}

// One wave per row writes the set bits of its mask in ascending order: the row's
// mask words are loaded 64 at a time, one per lane, and the non-zero ones visited
// in order, each set bit's lane writing its block.  With the sigma gate, rows of
// fired tiles add their expansion bits (disjoint from the kept bits) and the
// row's gate flag is its tile's decision.  CSR: the row's offset is its run's
// scanned offset plus the counts of the rows before it in the run (clamped to the
// capacity like the run offsets), written to row_ptr here.  With width > 0 the
// output is the padded list instead: row r occupies [r*width, (r+1)*width), its
// blocks ascending and then -1 sentinels, with no scan.
__global__ __launch_bounds__(256) void compact_kernel(const unsigned long long* __restrict__ mask,
                                                      const unsigned long long* __restrict__ mask_x,
                                                      const uint8_t* __restrict__ fire,
                                                      uint8_t* __restrict__ gate_out,
                                                      const int* __restrict__ counts,
                                                      const int32_t* __restrict__ run_off,
                                                      int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ col_idx, int rows,
                                                      int nb, int nw, int64_t capacity, int width,
                                                      int* __restrict__ overflow) {
  const int l = lane_id();
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = row % nb;
  const int nslots = i / 64 + 1;
  int64_t base;
  if (width > 0) {
    base = (int64_t)row * width;
    capacity = base + width;
  } else {
    const int r0 = row & ~63, k = row - r0;
    const int before = wave_sum_int(l < k ? counts[r0 + l] : 0);
    base = (int64_t)run_off[row >> 6] + before;
    if (l == 0) {
      row_ptr[row] = (int32_t)(base < capacity ? base : capacity);
      if (row == rows - 1) row_ptr[rows] = run_off[(rows + 63) >> 6];
    }
  }
  const bool expand = fire != nullptr && fire[i];
  if (fire != nullptr && gate_out != nullptr && l == 0) gate_out[row] = expand ? 1 : 0;
  int run = 0;
  const unsigned long long lt = lanemask_lt();
  const unsigned long long* mrow = mask + (size_t)row * nw;
  const unsigned long long* xrow = expand ? mask_x + (size_t)row * nw : nullptr;
  for (int e0 = 0; e0 < nslots; e0 += 64) {
    const int e = e0 + l;
    const unsigned long long mine = e < nslots ? (mrow[e] | (xrow ? xrow[e] : 0ull)) : 0ull;
    unsigned long long nz = __ballot(mine != 0ull);
    while (nz) {
      const int f = __builtin_ctzll(nz);
      nz &= nz - 1;
      const unsigned lo = __builtin_amdgcn_readlane((unsigned)mine, f);
      const unsigned hi = __builtin_amdgcn_readlane((unsigned)(mine >> 32), f);
      const unsigned long long w = ((unsigned long long)hi << 32) | lo;
      if ((w >> l) & 1ull) {
        const int64_t pos = base + run + __popcll(w & lt);
        if (pos < capacity) col_idx[pos] = (e0 + f) * 64 + l;
      }
      run += __popcll(w);
    }
  }
  if (width > 0) {
    for (int p = run + l; p < width; p += 64) col_idx[base + p] = -1;
    if (run > width && l == 0) *overflow = 1;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

SelectWorkspace select_workspace_layout(const Shape& sh, bool export_scores, bool sigma_gate) {
  SelectWorkspace w;
  const size_t rows = (size_t)sh.U() * sh.nb;
  const size_t nw = (size_t)(sh.nb + 63) / 64;
  size_t off = 0;
  w.scores_off = off;
  if (!export_scores) off += align256(rows * sh.nb * sizeof(float));
  w.mask_off = off;
  off += align256(rows * nw * sizeof(unsigned long long));
  w.counts_off = off;
  off += align256(rows * sizeof(int));
  w.overflow_off = off;
  off += 256;
  const size_t nrun = (rows + 63) / 64;
  w.run_sum_off = off;
  off += align256(nrun * sizeof(int));
  w.run_off_off = off;
  off += align256((nrun + 1) * sizeof(int));
  w.sigma_off = w.mask_x_off = w.counts_x_off = w.keys_off = w.fire_off = off;
  if (sigma_gate) {
    w.sigma_off = off;
    off += align256(rows * sizeof(float));
    w.mask_x_off = off;
    off += align256(rows * nw * sizeof(unsigned long long));
    w.counts_x_off = off;
    off += align256(rows * sizeof(int));
    w.keys_off = off;
    off += align256((size_t)sh.nb * sizeof(unsigned));
    w.fire_off = off;
    off += align256((size_t)sh.nb);
  }
  w.total = off;
  return w;
}

namespace {

// Slots per lane of the register form of the select kernel for rows of nb
// blocks (0: rows too long, the LDS form runs).
int select_slots(int nb, bool topk_only) {
  const int nw = (nb + 63) / 64;
  return nw <= 1 ? 1 : nw <= 2 ? 2 : nw <= 4 ? 4 : nw <= 8 ? 8 : nw <= 16 ? 16
         : nw <= 32 ? 32 : nw <= 64 ? 64 : (nw <= 128 && topk_only) ? 128 : 0;
}

// The LDS form keeps each of its waves' rows in LDS: the scores, and the
// rescue bounds and probabilities when those branches are on.
size_t lds_row_bytes(int nb, bool use_b, bool use_p) {
  return (size_t)((nb + 63) / 64) * 64 * sizeof(float) * (1 + (use_b ? 1 : 0) + (use_p ? 1 : 0));
}

int lds_form_waves(size_t row_bytes) {
  const size_t w = 65536 / row_bytes;
  return w < 1 ? 1 : (w > 4 ? 4 : (int)w);
}

constexpr size_t kLdsLimit = 160 * 1024;  // LDS of one CU on gfx950

}  // namespace

size_t select_lds_bytes(const Shape& sh, const SelectConfig& cfg) {
  const bool use_b = cfg.rescue_fraction > 0.0, use_p = cfg.mass_threshold > 0.0f;
  if (select_slots(sh.nb, !use_b && !use_p) > 0) return 0;
  const size_t row = lds_row_bytes(sh.nb, use_b, use_p);
  return (size_t)lds_form_waves(row) * row;
}

size_t select_lds_limit() { return kLdsLimit; }

// ---- scratch of the allocation-free selection entry point
//
// One fixed array per GPU, in place of a caller's workspace, for callers that
// cannot allocate device memory.  Each GPU the library runs on holds it until
// the process ends; every call on a GPU shares that GPU's copy (calls that
// overlap on one GPU race).  Nothing in it has to start zeroed: every word a
// selection reads back was written earlier in the same call.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t select_scratch_bytes() { return kScratchBytes; }

hipError_t select_scratch(void** ptr) {
  // device address of `scratch` on the current device, looked up once per device
  // (the array's name in host code is a host-side stand-in, not that address)
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_score_select(const Shape& sh, const SelectConfig& cfg, const float* q_centroid,
                               const float* q_norm, const float* k_centroid,
                               const float* k_radius, int32_t* row_ptr, int32_t* col_idx,
                               int64_t col_capacity, float* scores_out, float* bound_out,
                               uint8_t* gate_out, void* workspace, hipStream_t stream,
                               const float* scores_in, int width) {
  const bool sig = cfg.gate == 2 && cfg.top_k > 0;
  const SelectWorkspace w =
      select_workspace_layout(sh, scores_out != nullptr || scores_in != nullptr, cfg.gate == 2);
  unsigned char* ws = (unsigned char*)workspace;
  float* scores = scores_in ? const_cast<float*>(scores_in)  // read only below
                            : scores_out ? scores_out : (float*)(ws + w.scores_off);
  unsigned long long* mask = (unsigned long long*)(ws + w.mask_off);
  int* counts = (int*)(ws + w.counts_off);
  const int nb = sh.nb, U = sh.U(), rows = U * nb, nw = (nb + 63) / 64;
  const int NT = (nb + 127) / 128;  // score tiles per side

  hipError_t e = hipSuccess;
  // The LDS form beyond 64 KiB needs the kernel's dynamic LDS limit raised (once
  // per device); done before the first launch so that a failure launches nothing.
  const size_t lds_bytes = select_lds_bytes(sh, cfg);
  if (lds_bytes > kLdsLimit) return hipErrorInvalidValue;  // rejected by the caller first
  if (lds_bytes > 65536) {
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    (void)hipGetDevice(&dev);
    const uint64_t bit = 1ull << (dev & 63);
    if (!(attr_set.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute((const void*)select_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
      if (e != hipSuccess) return e;
      attr_set.fetch_or(bit, std::memory_order_acq_rel);
    }
  }
  if (!scores_in) {
    hipLaunchKernelGGL(score_kernel, dim3(NT * (NT + 1) / 2, U), dim3(256), 0, stream, q_centroid,
                       k_centroid, scores, nb, sh.D, sh.G(), sh.per_group);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  SelArgs a;
  a.scores = scores;
  a.qn = q_norm;
  a.kr = k_radius;
  a.bound_out = bound_out;
  a.gate_out = gate_out;
  a.mask = mask;
  a.counts = counts;
  a.nb = nb;
  a.nw = nw;
  a.rows = rows;
  a.units = nb > 0 ? rows / nb : 0;
  a.i0 = 0;
  a.ni = nb;
  a.G = sh.G();
  a.per_group = sh.per_group;
  a.top_k = cfg.top_k;
  a.force_sink = cfg.force_sink;
  a.gate = cfg.gate;
  a.gate_factor = cfg.gate_factor;
  a.gate_threshold = cfg.gate_threshold;
  a.tau_log2e = cfg.temperature * kLog2e;
  a.mass_threshold = cfg.mass_threshold;
  a.rescue_fraction = cfg.rescue_fraction;
  a.use_b = cfg.rescue_fraction > 0.0 ? 1 : 0;
  a.use_p = cfg.mass_threshold > 0.0f ? 1 : 0;
  a.per_wave_floats = nw * 64 * (1 + a.use_b + a.use_p);
  a.sigma = sig ? (float*)(ws + w.sigma_off) : nullptr;
  a.mask_x = sig ? (unsigned long long*)(ws + w.mask_x_off) : nullptr;
  a.counts_x = sig ? (int*)(ws + w.counts_x_off) : nullptr;
  a.overflow = (int*)(ws + w.overflow_off);
  // register form for rows up to 64*SPL = 4096 blocks (8192 with the top-k and
  // gate branches only), LDS form beyond.  When rows reach 64 slots the register
  // form runs once per range of query blocks [64*SPL/2, 64*SPL), each with the
  // fewest slots its rows need (rows below 1024 blocks share the 16-slot launch),
  // longest rows first; with the top-k and gate branches only, the 32- to 128-slot
  // forms leave out the rescue and mass state.
  const bool topk_only = !a.use_b && !a.use_p;
  const int spl = select_slots(nb, topk_only);
// one launch of the register form: N slots, FULL (every branch) or top-k only,
// the sigma gate's form when it is on
#define BSA_SELECT_REG(N, F)                                                          \
  if (sig)                                                                            \
    hipLaunchKernelGGL((select_reg_kernel<N, F, true>), rg, rb, 0, stream, a);        \
  else                                                                                \
    hipLaunchKernelGGL((select_reg_kernel<N, F, false>), rg, rb, 0, stream, a);       \
  break;
  if (spl > 0) {
    // (short layers, widest form below 64 slots: a single launch)
    const int smin = spl >= 64 ? 16 : spl;
    for (int s = spl; s >= smin; s /= 2) {
      const int lo = (s == smin) ? 0 : 64 * s / 2;
      const int hi = 64 * s < nb ? 64 * s : nb;
      if (lo >= hi) continue;
      a.i0 = lo;
      a.ni = hi - lo;
      const dim3 rg((unsigned)(((int64_t)a.units * a.ni + 3) / 4)), rb(256);
      const int form = (topk_only && s >= 32) ? -s : s;  // negative: top-k-only form
      switch (form) {
        case 1: BSA_SELECT_REG(1, true)
        case 2: BSA_SELECT_REG(2, true)
        case 4: BSA_SELECT_REG(4, true)
        case 8: BSA_SELECT_REG(8, true)
        case 16: BSA_SELECT_REG(16, true)
        case 32: BSA_SELECT_REG(32, true)
        case 64: BSA_SELECT_REG(64, true)
        case -32: BSA_SELECT_REG(32, false)
        case -64: BSA_SELECT_REG(64, false)
        case -128: BSA_SELECT_REG(128, false)
        default:
          return hipErrorInvalidValue;
      }
#undef BSA_SELECT_REG
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    const size_t per_wave_bytes = (size_t)a.per_wave_floats * sizeof(float);
    const int waves = lds_form_waves(per_wave_bytes);
    hipLaunchKernelGGL(select_kernel, dim3((rows + waves - 1) / waves), dim3(64 * waves),
                       lds_bytes, stream, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  uint8_t* fire = nullptr;
  if (sig) {
    fire = ws + w.fire_off;
    const int in_lds = nb <= 8192 ? 1 : 0;  // 32 KiB of keys
    hipLaunchKernelGGL(sigma_tile_kernel, dim3(1), dim3(1024), in_lds ? nb * sizeof(unsigned) : 0,
                       stream, a.sigma, (unsigned*)(ws + w.keys_off), fire, U, nb, cfg.top_k,
                       cfg.force_sink, cfg.gate_threshold, in_lds);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }  // (with the top-k branch off the select kernel writes gate_out = 0 itself)

  int* run_sum = (int*)(ws + w.run_sum_off);
  int32_t* run_off = (int32_t*)(ws + w.run_off_off);
  if (width == 0) {
    if (fire) {
      hipLaunchKernelGGL(expand_counts_kernel, dim3((rows + 255) / 256), dim3(256), 0, stream,
                         counts, a.counts_x, fire, rows, nb);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int nrun = (rows + 63) / 64;
    hipLaunchKernelGGL(run_sum_kernel, dim3((nrun + 3) / 4), dim3(256), 0, stream, counts,
                       run_sum, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, run_sum, run_off, nrun,
                       col_capacity, a.overflow);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(compact_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, mask, a.mask_x,
                     fire, gate_out, counts, run_off, row_ptr, col_idx, rows, nb, nw,
                     col_capacity, width, a.overflow);
  return hipGetLastError();
}

}  // namespace bsa
