// Block-sparse attention forward on the bf16 matrix cores of CDNA4 (gfx950).
//
// Method: each query block attends only over the key blocks its selection row
// kept, with the causal mask inside the diagonal block, as FlashAttention does
// over the fused sparse mask (RBS-Attention, third paragraph; MiniMax MSA,
// "What is MSA and how does it work": the main branch attends over the
// preselected blocks only).  Softmax is computed online, block by block.
//
// Work decomposition: one workgroup per (query head, query block); wave w (four
// waves at B = 128, two at B = 64) owns queries [32w, 32w + 32) against all B
// keys of every kept block and keeps its own running max, sum and output, so no
// partial results are merged.  The score tile is computed transposed,
// S^T = K Q^T, so that each lane holds one query column: the per-query max and
// sum are lane-local except for a single exchange between the two 32-lane
// halves (V_PERMLANE32_SWAP).  The probabilities then feed the second product
// O^T = V^T P^T straight from registers as the B operand, and the V^T operand is
// read from the row-major V tile with the gfx950 transposing LDS load
// (DS_READ_B64_TR_B16), so V is never transposed in memory.
//
// Memory and occupancy: a workgroup holds one K tile and one V tile in LDS
// (64 KiB at D = B = 128), filled by direct global->LDS DMA, so two workgroups
// share each CU: the two waves on a SIMD then belong to independent rows, and one
// row's set-up and memory waits are covered by the other's products.  Left alone
// the two waves fall into step (both in their products, then both in their
// softmax); a wave raises its priority from its row maximum through O += V P and
// lowers it for the next block's products, which keeps them out of phase (one's
// softmax on the VALU beside the other's products).  Within a
// block, K(n+1) streams in while O += V(n) P(n) runs, and V(n+1) while S(n+1)
// and its softmax run (two barriers per block).  LDS rows are XOR-swizzled in
// 16-byte chunks so that both the 16-byte K reads (32 rows, one column) and the
// transposing V reads (4 rows x 4 chunks per 32 lanes) are free of bank
// conflicts.  The grid is ordered kv-head major, by descending query block
// (longest rows first), and maps the heads of one GQA group at one query block
// to the same XCD, so their shared K/V blocks meet in the same L2.
//
// FP8 inputs (OCP E4M3): S^T = K Q^T runs on the gfx950 FP8 matrix cores
// (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with unit block scales: products of E4M3
// codes are exact in fp32, so this is the bf16 result at twice the rate), with K
// read raw from LDS and Q held raw in registers; V is expanded to bf16 in LDS
// (exact) for O^T = V^T P^T.  q_scale and k_scale fold into the per-block logit
// scale and v_scale into the exponent of the probabilities.  When the caller has
// expanded the V codes to bf16 beforehand (exactly, with the library's expansion
// kernel), the V tiles are copied straight into LDS as bf16 and the per-block
// expansion and its barrier drop out; the results are the same bit for bit.
#include <atomic>

#include "common.h"
#include "launch.h"

namespace bsa {

namespace {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const int32_t* row_ptr;  // CSR rows, or nullptr with the padded list
  const int32_t* col_idx;
  void* out;
  float* lse;
  int64_t S;
  int Hq, Hkv, nb, per_group;
  int width;  // > 0: padded list, row r at col_idx[r*width], valid entries first
  float scale_log2;
};

// XOR applied to the 16-byte chunk index of LDS row r, shared by the K and V
// tiles; it depends on r mod 16 only.  D = 128 (256-byte rows, 16 chunks): the
// 16 rows of one chunk column (the 16-byte K operand reads) land on 16 distinct
// chunks of the 256-byte bank window, and any 4 consecutive rows are moved to
// 4 different 4-chunk groups, so a transposing V read (4 rows x 4 chunks over
// 32 lanes) touches every bank once.  D = 64 (128-byte rows, two per window):
// the same two properties among the rows of one parity.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  const int k = (r >> 1) & 7;
  return ((k & 1) << 2) | (k >> 1);
}
// Raw E4M3 tiles (rows of D bytes, 16-byte chunks c): XOR applied to the chunk
// index so that the 16 rows of one chunk column sit on 16 distinct 16-byte
// slots of the 256-byte bank window (D = 128: two rows per window; D = 64: four).
template <int D>
__device__ __forceinline__ int swz8(int r) {
  return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  return r * (D * 2) + ((c ^ swz<D>(r)) << 4);
}
template <int D>
__device__ __forceinline__ int v_off(int r, int c) {
  return k_off<D>(r, c);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// ---- staging: global -> LDS by direct-to-LDS DMA (GLOBAL_LOAD_LDS_DWORDX4).
// One DMA instruction moves 64 lanes x 16 bytes into 1 KiB of LDS at M0, lane
// L landing at byte 16L; the swizzle is applied by choosing which global chunk
// lane L fetches.  The loads are issued from inline asm (they have no register
// results) so that the compiler does not serialise them against the LDS reads
// of the other tile; completion is awaited explicitly (S_WAITCNT vmcnt) before
// the workgroup barrier.

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from sbase + voff (SADDR form: uniform 64-bit base in SGPRs,
// 32-bit per-lane byte offset) into LDS at M0 + 16 * lane.
__device__ __forceinline__ void dma16(const void* sbase, unsigned voff, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until no vector-memory operation of this wave is outstanding.  This is
// the S_WAITCNT builtin (vmcnt 0, expcnt and lgkmcnt left open) rather than
// inline asm, so the compiler sees the wait and knows every earlier vector load
// has completed; otherwise it keeps ordinary loads issued before the loop (the
// Q fragments) pending and waits on vmcnt inside the loop, which, counting the
// DMAs it cannot see, would stall on the next block's transfer.
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding: vmcnt(0) expcnt(7) lgkmcnt(15)
}

// Workgroup barrier that also completes this wave's LDS accesses.  The builtin
// wait tells the compiler that nothing counted by lgkmcnt is outstanding (a
// pending scalar load would otherwise force every later LDS wait down to zero);
// the asm repeats it next to the barrier, and its memory clobber keeps the
// compiler from moving loads or stores across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: vmcnt(63) expcnt(7) lgkmcnt(0)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, int B>
struct WCfg {
  static constexpr int NW = B / 32;    // waves = 32-query groups
  static constexpr int NT = 64 * NW;
  static constexpr int NKT = B / 32;   // 32-key tiles per block
  static constexpr int NDS = D / 16;
  static constexpr int NDT = D / 32;
  static constexpr int ROWB = D * 2;
  static constexpr int TILE = B * ROWB;
};

// exp2 of key tile kt2: p = 2^(s*sl - m), summed per query, scaled by vsc (E4M3
// value scale) and packed to the bf16 B operands of its two 16-key steps.
__device__ __forceinline__ void probs(const f32x16& s, float nref, float sl, float vsc, float& psum,
                                      u32x4 (&pk)[2]) {
  float p[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    p[v] = __builtin_amdgcn_exp2f(fmaf(s[v], sl, nref));
    psum += p[v];
  }
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pk[sb][e] = pack_bf16x2(p[8 * sb + 2 * e] * vsc, p[8 * sb + 2 * e + 1] * vsc);
}

// O^T += V^T P^T over the two 16-key steps of key tile kt2.  The key rows of one
// step are 4*hf + [0,4) (elements 0..3) and the same + 8 (elements 4..7); their
// swizzle does not depend on the step, so the step offset folds into the read.
template <int D, int B>
__device__ __forceinline__ void pv_tile(const unsigned char* vrow, const u32x4 (&pk)[2],
                                        f32x16 (&o)[D / 32], int kt2, int rlo, int cb0) {
  typedef WCfg<D, B> C;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int step = (kt2 * 32 + sb * 16) * C::ROWB;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const int c = (dt * 64 + cb0) >> 4;  // chunk of this lane's 8 bytes
      const s16x4 lo = lds_read_tr16(vrow + step + ((c ^ swz<D>(rlo)) << 4));
      const s16x4 hi = lds_read_tr16(vrow + 8 * C::ROWB + step + ((c ^ swz<D>(rlo + 8)) << 4));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pk[sb]),
                                                      o[dt], 0, 0, 0);
    }
  }
}

// Transposed V tiles (bsa_prepare_v's layout, D = B = 128): row d of the tile holds
// dimension d of the block's keys, each 16-key group stored in the order
// 0-3, 8-11, 4-7, 12-15, which is the order in which the probabilities sit in the
// B operand (lane half hf holds keys 4hf + {0..3, 8..11} of each 16-key step).  So
// the V^T operand of a step is one 16-byte read: row l % 32 (+ 32 dt), chunk
// 4 kt2 + 2 sb + hf, behind the K tiles' swizzle (same 256-byte rows).
template <int D, int B>
__device__ __forceinline__ void pv_tile_t(const unsigned char* vtile, const u32x4 (&pk)[2],
                                          f32x16 (&o)[D / 32], int kt2, int l) {
  typedef WCfg<D, B> C;
  static_assert(D == 128 && B == 128, "transposed V tiles are 128 x 128");
  const int row = l & 31, hf = l >> 5, sw = swz<D>(row);
  const unsigned char* rp = vtile + row * (B * 2);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int chunk = 4 * kt2 + 2 * sb + hf;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const bf16x8 vf = *(const bf16x8*)(rp + dt * 32 * (B * 2) + ((chunk ^ sw) << 4));
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pk[sb]),
                                                      o[dt], 0, 0, 0);
    }
  }
}

// DMA of one transposed V tile: [D][B] bf16, contiguous for block j and kv head g
// at ((j * Hkv + g) * D) * B; rows of 2B bytes land swizzled like the K tiles.
template <int D, int B>
struct VtTiles {
  static constexpr int NW = B / 32;
  static constexpr int ROW = B * 2;
  static constexpr int TILE = D * ROW;
  static constexpr int NI = TILE / (1024 * NW);
  static_assert(NI >= 1 && TILE % (1024 * NW) == 0, "tile must split into 1 KiB DMAs");

  static __device__ __forceinline__ void plan(int wave, int l, unsigned* off) {
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int p = (wave * NI + n) * 1024 + 16 * l;
      const int r = p / ROW;
      off[n] = (unsigned)(r * ROW + ((((p % ROW) >> 4) ^ swz<D>(r)) << 4));
    }
  }
  static __device__ __forceinline__ void issue(const void* src, int Hkv, int g, int j,
                                               unsigned char* dst, int wave, const unsigned* off) {
    const unsigned char* base = (const unsigned char*)src + ((size_t)j * Hkv + g) * TILE;
#pragma unroll
    for (int n = 0; n < NI; ++n) dma16(base, off[n], lds_addr(dst + (wave * NI + n) * 1024));
  }
};

// ---------------------------------------------------------------------------
// Tiles of one workgroup and the order of one block's work:
//   S(n), P(n) | wait V(n), barrier | request K(n+1) | O += V(n) P(n) |
//   wait K(n+1), barrier | request V(n+1)

template <int D, int B, bool FP8>
struct WTiles {
  typedef WCfg<D, B> C;
  static constexpr int RAW_TILE = FP8 ? B * D : C::TILE;
  static constexpr int NI = RAW_TILE / (1024 * C::NW);  // DMA instructions per wave per tile
  static constexpr int KBUF = 0, VBUF = RAW_TILE, XV = 2 * RAW_TILE;
  static constexpr int LDS_BYTES = FP8 ? 2 * RAW_TILE + C::TILE : 2 * C::TILE;
  static_assert(NI >= 1 && RAW_TILE % (1024 * C::NW) == 0, "tile must split into 1 KiB DMAs");

  static __device__ __forceinline__ void plan(const AttnArgs& a, int wave, int l, unsigned* off) {
    constexpr int ES = FP8 ? 1 : 2;
    const unsigned rs = (unsigned)(a.Hkv * D * ES);
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int p = (wave * NI + n) * 1024 + 16 * l;
      int r, col;
      if (!FP8) {
        r = p / C::ROWB;
        col = (((p % C::ROWB) >> 4) ^ swz<D>(r)) << 4;
      } else {
        r = p / D;
        col = (((p % D) >> 4) ^ swz8<D>(r)) << 4;
      }
      off[n] = (unsigned)r * rs + (unsigned)col;
    }
  }

  // this wave's share of tile `src` (K or V) of key block j into `dst`; rows past
  // the ragged end re-read the last row (their logits are masked)
  static __device__ __forceinline__ void issue(const AttnArgs& a, const void* src, int g, int j,
                                               unsigned char* dst, int wave, const unsigned* off) {
    constexpr int ES = FP8 ? 1 : 2;
    const unsigned char* base =
        (const unsigned char*)src + ((size_t)j * B * a.Hkv + (size_t)g) * D * ES;
    const int64_t left = a.S - (int64_t)j * B;
    if (left >= B) {
#pragma unroll
      for (int n = 0; n < NI; ++n) dma16(base, off[n], lds_addr(dst + (wave * NI + n) * 1024));
    } else {
      const unsigned rs = (unsigned)(a.Hkv * D * ES);
      const unsigned last = (unsigned)(left - 1) * rs;
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const unsigned col = off[n] % rs, rowoff = off[n] - col;
        dma16(base, (rowoff < last ? rowoff : last) + col, lds_addr(dst + (wave * NI + n) * 1024));
      }
    }
  }

  static __device__ __forceinline__ void expand_v(const unsigned char* raw, unsigned char* vt,
                                                  int tid) {
    constexpr int NC8 = D / 16;
    constexpr int PER = B * NC8 / C::NT;
    static_assert(PER >= 1 && B * NC8 % C::NT == 0, "expand split");
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int ci = tid + C::NT * n;
      const int r = ci / NC8, c = ci % NC8;
      const u32x4 w = *(const u32x4*)(raw + r * D + ((c ^ swz8<D>(r)) << 4));
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x2 x0 = e4m3x4_to_bf16x4(w[2 * hh]), x1 = e4m3x4_to_bf16x4(w[2 * hh + 1]);
        *(u32x4*)(vt + v_off<D>(r, 2 * c + hh)) = u32x4{x0[0], x0[1], x1[0], x1[1]};
      }
    }
  }
};

template <int D, int B, bool FP8, bool V16, bool VT>
__global__ __launch_bounds__(64 * (B / 32), 2) void attn_whole_kernel(AttnArgs a) {
  typedef WCfg<D, B> C;
  typedef WTiles<D, B, FP8> ST;
  typedef WTiles<D, B, false> SV;  // V tiles given as bf16 (E4M3 codes expanded beforehand)
  typedef VtTiles<D, B> TV;        // V tiles given transposed (bsa_prepare_v)
  static_assert(!V16 || FP8, "bf16 V is the E4M3 path's option");
  static_assert(!VT || (D == 128 && B == 128 && (V16 || !FP8)), "transposed V: 128 x 128 bf16");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = l >> 5;

  // work order: kv-head major (the whole chip works through one kv head's K/V at
  // a time, a working set that stays resident in the last-level cache), longest
  // query block first within a kv head, and the heads of one group at one query
  // block on one XCD (workgroup id mod 8), so their common K/V blocks meet in one L2
  const int G = a.Hq / a.Hkv, nb = a.nb;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, t8 = bid >> 3;
  const int hh = t8 % G;
  const int r = (t8 / G) * 8 + xcd;
  if (r >= a.Hkv * nb) return;  // padding workgroup (uniform: no barrier reached)
  const int g = r / nb, i = nb - 1 - r % nb;
  const int h = g * G + hh;
  const int unit = a.per_group ? g : h;
  const int row = unit * nb + i;
  int e0, nblk;
  if (a.width > 0) {
    // padded row: its valid entries (a prefix of the row) are counted by ballots
    e0 = row * a.width;
    nblk = 0;
    for (int c = 0; c < a.width; c += 64)
      nblk += __popcll(__ballot(c + l < a.width && a.col_idx[e0 + c + l] >= 0));
  } else {
    e0 = a.row_ptr[row];
    nblk = a.row_ptr[row + 1] - e0;
  }

  // kept block ids (and E4M3 scales) 64 at a time, lane L holding entry base + L,
  // read back with V_READLANE; -1 marks an entry outside the causal range, whose
  // block is loaded (block 0) but fully masked
  int cbase = 0, cid = -1;
  float cks = 1.f, cvs = 1.f;
  auto load_chunk = [&](int base) {
    cbase = base;
    const int n = base + l;
    const int j = n < nblk ? a.col_idx[e0 + n] : -1;
    cid = (j >= 0 && j <= i) ? j : -1;
    if (FP8) {
      const size_t o = (size_t)g * nb + (cid < 0 ? 0 : cid);
      cks = a.k_scale[o];
      cvs = a.v_scale[o];
    }
  };
  auto id_at = [&](int n) { return __builtin_amdgcn_readlane(cid, n - cbase); };
  auto blk = [](int j) { return j < 0 ? 0 : j; };
  unsigned doff[ST::NI];
  ST::plan(a, wave, l, doff);
  unsigned voff[VT ? TV::NI : V16 ? SV::NI : 1];
  if constexpr (VT)
    TV::plan(wave, l, voff);
  else if (V16)
    SV::plan(a, wave, l, voff);
  // V(j): raw tile (then expanded in LDS), or the bf16 tile straight into place,
  // or the transposed bf16 tile
  auto issue_v = [&](int j) {
    if constexpr (VT)
      TV::issue(a.v, a.Hkv, g, j, lds + (FP8 ? ST::XV : ST::VBUF), wave, voff);
    else if (V16)
      SV::issue(a, a.v, g, j, lds + ST::XV, wave, voff);
    else
      ST::issue(a, a.v, g, j, lds + ST::VBUF, wave, doff);
  };
  if (nblk > 0) {
    load_chunk(0);
    const int j0 = blk(id_at(0));
    ST::issue(a, a.k, g, j0, lds + ST::KBUF, wave, doff);
    issue_v(j0);
  }

  // ---- Q fragments (B operand of S^T = K Q^T), query column = lane % 32.
  // bf16: contraction index d = ds*16 + hf*8 + [0, 8) of step ds.  E4M3: byte b
  // of product mm is d = mm*64 + hf*32 + b, the same assignment the K operand
  // reads use (any common assignment of the contraction index to operand bytes
  // gives the same product).
  bf16x8 qf[FP8 ? 1 : C::NDS];
  i32x8 qf8[FP8 ? D / 64 : 1];
  const float qsc = FP8 ? a.q_scale[(size_t)h * nb + i] : 1.0f;
  const int qi = wave * 32 + (l & 31);
  {
    int64_t t = (int64_t)i * B + qi;
    t = t < a.S ? t : a.S - 1;
    if (!FP8) {
#pragma unroll
      for (int ds = 0; ds < C::NDS; ++ds) {
        const size_t off = ((size_t)t * a.Hq + h) * D + ds * 16 + hf * 8;
        qf[ds] = __builtin_bit_cast(bf16x8, *(const u32x4*)((const uint16_t*)a.q + off));
      }
    } else {
#pragma unroll
      for (int mm = 0; mm < D / 64; ++mm) {
        const uint8_t* src = (const uint8_t*)a.q + ((size_t)t * a.Hq + h) * D + mm * 64 + hf * 32;
        const u32x4 lo = *(const u32x4*)src, hi = *(const u32x4*)(src + 16);
        qf8[mm] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
    }
  }

  f32x16 o[C::NDT];
  float m = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) o[dt] = f32x16{0};

  const int kx = hf ^ swz<D>(l & 31);
  const int rlo = 4 * hf + ((l & 15) >> 2);
  const int cb0 = (((l >> 4) & 1) * 16 + 4 * (l & 3)) * 2;
  const int kfirst = hf * 4;
  const int vrow0 = rlo * C::ROWB + (cb0 & 15);

  wait_vmem_all();
  lds_barrier();
  for (int n = 0; n < nblk; ++n) {
    const int j = id_at(n);
    const float ksc =
        FP8 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cks), n - cbase)) : 1.0f;
    const float vsc =
        FP8 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cvs), n - cbase)) : 1.0f;
    int jn = 0;
    if (n + 1 < nblk) {
      if (n + 1 - cbase >= 64) load_chunk(cbase + 64);
      jn = blk(id_at(n + 1));
    }

    // ---- S^T = K(n) Q^T and the online softmax (K(n) is in LDS)
    f32x16 s[C::NKT];
#pragma unroll
    for (int kt2 = 0; kt2 < C::NKT; ++kt2) s[kt2] = f32x16{0};
    if (!FP8) {
      // the K fragments of step ds + 1 are requested before the products of step
      // ds (the scheduling barriers keep that order), one step of latency hidden
      const unsigned char* krow = lds + ST::KBUF + (l & 31) * C::ROWB;
      bf16x8 kf[2][C::NKT];
#pragma unroll
      for (int kt2 = 0; kt2 < C::NKT; ++kt2)
        kf[0][kt2] = *(const bf16x8*)(krow + (kx << 4) + kt2 * 32 * C::ROWB);
#pragma unroll
      for (int ds = 0; ds < C::NDS; ++ds) {
        if (ds + 1 < C::NDS) {
          const unsigned char* ka = krow + (((2 * (ds + 1)) ^ kx) << 4);
#pragma unroll
          for (int kt2 = 0; kt2 < C::NKT; ++kt2)
            kf[(ds + 1) & 1][kt2] = *(const bf16x8*)(ka + kt2 * 32 * C::ROWB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt2 = 0; kt2 < C::NKT; ++kt2)
          s[kt2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds & 1][kt2], qf[ds], s[kt2], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      const unsigned char* krow = lds + ST::KBUF + (l & 31) * D;
      const int sw = swz8<D>(l & 31);
#pragma unroll
      for (int mm = 0; mm < D / 64; ++mm) {
        const int c0 = 4 * mm + 2 * hf;
        i32x8 kf8[C::NKT];
#pragma unroll
        for (int kt2 = 0; kt2 < C::NKT; ++kt2) {
          const unsigned char* rp = krow + kt2 * 32 * D;
          const u32x4 lo = *(const u32x4*)(rp + ((c0 ^ sw) << 4));
          const u32x4 hi = *(const u32x4*)(rp + (((c0 + 1) ^ sw) << 4));
          kf8[kt2] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int kt2 = 0; kt2 < C::NKT; ++kt2)
          s[kt2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf8[kt2], qf8[mm], s[kt2], 0, 0,
                                                                   0, 127, 0, 127);
      }
    }
    // Wave priority: the two waves on a SIMD run the same phases and, left to
    // themselves, fall into step, so that their products and their softmax
    // arithmetic serialise.  From the row maximum through O += V P this wave asks
    // for the issue slots first; for the next block's request and products it
    // yields, so a wave in its softmax runs ahead of one in its products.
    __builtin_amdgcn_s_setprio(2);
    // (an all-zero E4M3 block has scale 0: its logits are all zero, and a floor
    // of 1e-30 on the logit scale keeps them so, to within 1e-22, while masked
    // keys stay at -inf instead of becoming -inf * 0 = NaN)
    const float sl = fmaxf(a.scale_log2 * qsc * ksc, 1e-30f);
    float mx = -INFINITY;
    if (j < 0 || j == i || (int64_t)j * B + B > a.S) {
      int lim = -1;
      if (j >= 0) {
        const int64_t left = a.S - (int64_t)j * B - 1 - kfirst;
        lim = (int)(left < 4 * B ? left : 4 * B);
        if (j == i) lim = min(lim, qi - kfirst);
      }
#pragma unroll
      for (int kt2 = 0; kt2 < C::NKT; ++kt2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kw = kt2 * 32 + (v >> 2) * 8 + (v & 3);
          const float x = kw > lim ? -INFINITY : s[kt2][v];
          s[kt2][v] = x;
          mx = fmaxf(mx, x);
        }
    } else {
#pragma unroll
      for (int kt2 = 0; kt2 < C::NKT; ++kt2)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt2][v]);
    }
    mx = max_with_other_half(mx) * sl;
    const bool bump = mx > m + 8.0f;
    if (__ballot(bump)) {
      const float alpha = bump ? __builtin_amdgcn_exp2f(m - mx) : 1.0f;
      m = bump ? mx : m;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
    }
    const float nref = m == -INFINITY ? 0.f : -m;
    float psum = 0.f;
    u32x4 pk[C::NKT][2];
    if (FP8) {
      // the block's value scale enters the exponent, p * vsc = 2^(x + log2 vsc), so
      // the probabilities need no multiply and their sum is divided by vsc once; a
      // zero scale (an all-zero block) is floored at 1e-30, whose products with the
      // codes are negligible, and the sum still counts the block's keys
      const float vs = fmaxf(vsc, 1e-30f);
      const float nv = nref + __builtin_amdgcn_logf(vs);
#pragma unroll
      for (int kt2 = 0; kt2 < C::NKT; ++kt2) probs(s[kt2], nv, sl, 1.0f, psum, pk[kt2]);
      psum *= __builtin_amdgcn_rcpf(vs);
    } else {
#pragma unroll
      for (int kt2 = 0; kt2 < C::NKT; ++kt2) probs(s[kt2], nref, sl, vsc, psum, pk[kt2]);
    }
    lsum += psum;

    // ---- V(n) has landed everywhere and K(n) is free: request K(n + 1)
    wait_vmem_all();
    lds_barrier();
    if (n + 1 < nblk) ST::issue(a, a.k, g, jn, lds + ST::KBUF, wave, doff);
    const unsigned char* vt = lds + ST::VBUF;
    if (FP8 && !V16) {
      ST::expand_v(lds + ST::VBUF, lds + ST::XV, tid);
      lds_barrier();
    }
    if (FP8) vt = lds + ST::XV;
    if constexpr (VT) {
#pragma unroll
      for (int kt2 = 0; kt2 < C::NKT; ++kt2) pv_tile_t<D, B>(vt, pk[kt2], o, kt2, l);
    } else {
#pragma unroll
      for (int kt2 = 0; kt2 < C::NKT; ++kt2) pv_tile<D, B>(vt + vrow0, pk[kt2], o, kt2, rlo, cb0);
    }

    // ---- K(n + 1) has landed everywhere and V(n) is free: request V(n + 1)
    __builtin_amdgcn_s_setprio(0);
    wait_vmem_all();
    lds_barrier();
    if (n + 1 < nblk) issue_v(jn);
  }

  // ---- output: this wave owns its 32 queries outright
  lsum += other_half(lsum);
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  const int64_t t = (int64_t)i * B + qi;
  if (t < a.S) {
    uint16_t* orow = (uint16_t*)a.out + ((size_t)t * a.Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int d = dt * 32 + vg * 8 + hf * 4;
        *(u32x2*)(orow + d) = u32x2{pack_bf16x2(o[dt][4 * vg] * inv, o[dt][4 * vg + 1] * inv),
                                    pack_bf16x2(o[dt][4 * vg + 2] * inv, o[dt][4 * vg + 3] * inv)};
      }
    if (a.lse && hf == 0)
      a.lse[(size_t)h * a.S + t] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
  }
}

template <int D, int B, bool FP8, bool V16 = false, bool VT = false>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  typedef WTiles<D, B, FP8> WT;
  static_assert(WT::LDS_BYTES <= 80 * 1024, "two workgroups per CU must fit the 160 KiB LDS");
  const int G = a.Hq / a.Hkv;
  const int rows8 = (a.Hkv * a.nb + 7) / 8;
  // the LDS limit is raised once per device (64 KiB and more need the attribute)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    const hipError_t e = hipFuncSetAttribute((const void*)attn_whole_kernel<D, B, FP8, V16, VT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             WT::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((attn_whole_kernel<D, B, FP8, V16, VT>), dim3(rows8 * 8 * G), dim3(WCfg<D, B>::NT),
                     WT::LDS_BYTES, stream, a);
  return hipGetLastError();
}

// E4M3 codes -> bf16, exactly (every E4M3 value is a bf16 value): 16 codes per
// thread, one 16-byte load and two 16-byte stores.
__global__ __launch_bounds__(256) void expand_e4m3_kernel(const u32x4* __restrict__ codes,
                                                          u32x4* __restrict__ out, int64_t n16) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n16) return;
  const u32x4 w = codes[t];
  const u32x2 a = e4m3x4_to_bf16x4(w[0]), b = e4m3x4_to_bf16x4(w[1]);
  const u32x2 c = e4m3x4_to_bf16x4(w[2]), d = e4m3x4_to_bf16x4(w[3]);
  out[2 * t] = u32x4{a[0], a[1], b[0], b[1]};
  out[2 * t + 1] = u32x4{c[0], c[1], d[0], d[1]};
}

// V [S, Hkv, 128] (bf16, or E4M3 codes expanded exactly) -> transposed bf16 tiles
// [nb, Hkv, 128 dims, 128 keys], each 16-key group in the order 0-3, 8-11, 4-7,
// 12-15 (the probabilities' order in the PV products), keys past S zero.  One
// workgroup per (block, kv head): the tile's rows are loaded with 16-byte (8-byte
// for codes) coalesced loads into LDS, then each thread gathers 8 keys of one
// dimension and writes them as one 16-byte store, 16 threads per 256-byte row.
template <bool FP8>
__global__ __launch_bounds__(256) void prepare_v_kernel(const void* __restrict__ v,
                                                        uint16_t* __restrict__ vt, int64_t S,
                                                        int Hkv) {
  constexpr int D = 128, B = 128, P = D + 2;  // padded LDS row (elements)
  __shared__ uint16_t ts[B * P];
  const int j = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int idx = it * 256 + tid, kk = idx >> 4, c = idx & 15;
    const int64_t t = (int64_t)j * B + kk;
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (t < S) {
      if (FP8) {
        const u32x2 codes =
            *(const u32x2*)((const uint8_t*)v + ((size_t)t * Hkv + g) * D + c * 8);
        const u32x2 a = e4m3x4_to_bf16x4(codes[0]), b = e4m3x4_to_bf16x4(codes[1]);
        w = u32x4{a[0], a[1], b[0], b[1]};
      } else {
        w = *(const u32x4*)((const uint16_t*)v + ((size_t)t * Hkv + g) * D + c * 8);
      }
    }
    uint16_t* dst = ts + kk * P + c * 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      dst[2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int idx = it * 256 + tid, d = idx >> 4, oc = idx & 15;
    const int k0 = 16 * (oc >> 1) + 4 * (oc & 1);  // keys k0 + {0..3, 8..11}
    unsigned y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ka = k0 + (e < 2 ? 2 * e : 2 * e + 4);
      y[e] = (unsigned)ts[ka * P + d] | ((unsigned)ts[(ka + 1) * P + d] << 16);
    }
    *(u32x4*)(vt + (((size_t)j * Hkv + g) * D + d) * B + oc * 8) = u32x4{y[0], y[1], y[2], y[3]};
  }
}

}  // namespace

hipError_t launch_prepare_v(const Shape& sh, const void* v, void* vt, hipStream_t stream) {
  if (sh.D != 128 || sh.B != 128) return hipErrorInvalidValue;
  if (sh.nb == 0) return hipSuccess;
  const dim3 grid((unsigned)sh.nb, (unsigned)sh.Hkv);
  if (sh.fp8)
    hipLaunchKernelGGL(prepare_v_kernel<true>, grid, dim3(256), 0, stream, v, (uint16_t*)vt, sh.S,
                       sh.Hkv);
  else
    hipLaunchKernelGGL(prepare_v_kernel<false>, grid, dim3(256), 0, stream, v, (uint16_t*)vt,
                       sh.S, sh.Hkv);
  return hipGetLastError();
}

hipError_t launch_expand_e4m3(const Shape& sh, const void* codes, void* out, hipStream_t stream) {
  const int64_t n16 = sh.S * sh.Hkv * sh.D / 16;  // D is a multiple of 16
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(expand_e4m3_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream,
                     (const u32x4*)codes, (u32x4*)out, n16);
  return hipGetLastError();
}

hipError_t launch_attention(const Shape& sh, const void* q, const void* k, const void* v,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            const int32_t* row_ptr, const int32_t* col_idx, float softmax_scale,
                            void* out, float* lse, hipStream_t stream, int width, bool v16,
                            bool vt) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.out = out;
  a.lse = lse;
  a.S = sh.S;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.nb = sh.nb;
  a.per_group = sh.per_group;
  a.width = width;
  a.scale_log2 = softmax_scale * kLog2e;
  if (vt) {
    if (sh.D != 128 || sh.B != 128) return hipErrorInvalidValue;
    return sh.fp8 ? launch_t<128, 128, true, true, true>(a, stream)
                  : launch_t<128, 128, false, false, true>(a, stream);
  }
#define BSA_ATTN(DD, BB)                                                               \
  if (sh.D == DD && sh.B == BB)                                                       \
    return !sh.fp8 ? launch_t<DD, BB, false>(a, stream)                                \
                   : v16 ? launch_t<DD, BB, true, true>(a, stream)                     \
                         : launch_t<DD, BB, true>(a, stream);
  BSA_ATTN(128, 128)
  BSA_ATTN(128, 64)
  BSA_ATTN(64, 64)
  BSA_ATTN(64, 128)
#undef BSA_ATTN
  return hipErrorInvalidValue;
}

}  // namespace bsa
