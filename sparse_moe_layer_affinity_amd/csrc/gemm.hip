// Grouped expert GEMMs of the MoE layer on gfx950.
//
// "DeepSeek-V3 Technical Report 深度解读报告", section 2.2: every token passes the
// shared expert(s) and its K routed experts; each expert is a SwiGLU FFN
// W_down (silu(W_gate u) * (W_up u)).  Rows are grouped by expert (see permute),
// the shared experts appended as groups E..E+Ns-1 holding all T tokens, so the
// whole layer is two grouped GEMMs:
//   GEMM1  h[r]      = silu(x[tok(r)] W_gate,e^T) * (x[tok(r)] W_up,e^T)   (gather on load)
//   GEMM2  y_rows[r] = h[r] W_down,e^T
// Both operands are K-contiguous (x and h rows, weight rows), which is exactly the
// operand layout of the MFMA: no transposes anywhere.
//
// One kernel, grouped_gemm_dma (below: row blocks of up to 320 rows, operands loaded
// straight into LDS), runs both expert GEMMs and the router logits (one group of T
// rows, fp32 split-K partials).  GEMM1's B tile stacks 128 gate rows over the
// matching 128 up rows and every wave owns the same columns of both halves, so the
// SwiGLU epilogue runs in registers; accumulation is fp32.

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gemm_common.h"

namespace moe {

// ---- LDS-DMA pipelined kernel for the expert GEMMs ---------------------------
// Tile: up to 320 rows (one expert's whole row block in the common case: about
// T*K/E = 256 rows, a few dozen more for the busier experts) x 256 output columns.
// Four waves each own a 128 x 128 block of the first 256 rows (4 x 4 MFMA 32x32x16
// accumulators in AGPRs) and a 32 x 128 strip of rows 256..319 (4 more accumulators
// in VGPRs, skipped when the tile has no such rows).  Covering up to 320 rows keeps
// the weights of an n-tile to one pass over HBM; a second, nearly empty 256-row tile
// would stream them again.
// Operands go global -> LDS directly with buffer loads in LDS mode ("buffer_load_dwordx4
// ... lds": lane i's 16 bytes land at M0 + 16 i): no registers stage them and no
// LDS-write instructions are issued.  K advances 64 per stage (a full 128-byte line of
// every row).  A (activations, mostly L2 hits: the n-tiles of a row block run side by
// side on one XCD) has two 40 KB stage buffers; B (weights, streamed from HBM) two of
// 32 KB.  Every B fragment of a stage is read into registers right after the stage is
// published; a second barrier then frees its buffer for the stage after next, so B
// stage k+2 streams while stage k is multiplied.  The loads are issued from inline
// assembly so the compiler does not fence them; each wave's own s_waitcnt vmcnt(n)
// before the barrier publishes a stage.
// LDS rows are 128 bytes (8 chunks); chunk c of row r sits in slot
// c ^ (r & 7) ^ ((r >> 3) & 1), conflict-free for the 16-lane groups of 128-bit
// fragment reads.  Lane p of DMA instruction j writes slot p & 7 of row 8 j + (p >> 3)
// of the wave's share, so it fetches chunk (p & 7) ^ (p >> 3) ^ (j & 1).
// Calls mf(m) for m in [MB, ME), with rd(q) for q < NRD and dm(q) for q < NDM spread
// evenly between them; the order is pinned (the scheduler would otherwise bunch the
// fragment reads and wait on each).
template <int MB, int ME, int NRD, int NDM, class MF, class RD, class DM>
__device__ __forceinline__ void interleave(MF&& mf, RD&& rd, DM&& dm) {
  constexpr int NS = ME - MB > 0 ? ME - MB : 1;
  static_for<0, NS>([&](auto q_tag) __attribute__((always_inline)) {
    constexpr int q = decltype(q_tag)::value;
    if constexpr (ME - MB > 0) mf(std::integral_constant<int, MB + q>{});
    __builtin_amdgcn_sched_barrier(0);
    static_for<q * NRD / NS, (q + 1) * NRD / NS>(rd);
    static_for<q * NDM / NS, (q + 1) * NDM / NS>(dm);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// MFMA with its accumulator in VGPRs.  The compiler gives every MFMA builtin an
// AGPR accumulator; a 320-row tile needs 320 accumulator registers per lane, the 64
// beyond the AGPR file in VGPRs, so the extra strip's MFMAs are written out.  Each
// such accumulator is reused only 16 or more MFMAs later; mfma_vgpr_drain covers the
// result latency before the first VALU read.
// The first MFMA of a chain takes an inline zero as SrcC: a VALU write of the
// accumulator just before an MFMA that reads it would need wait states the compiler
// does not insert around inline assembly.
__device__ __forceinline__ void mfma_vgpr(f32x16_t& c, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_first(f32x16_t& c, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_drain(f32x16_t* c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]));
}

// SHORT_K: K = 128 (two stages) only; otherwise K >= 256 (for split-K: every split).
// The two-stage sequence is compiled apart from the K loop: in one function it makes
// the register allocator spill around the loop.
template <int MODE, bool SHORT_K>
__global__ __launch_bounds__(256) void grouped_gemm_dma(GemmArgs a) {
  constexpr int BM = kExpertBM, BMAIN = 256, BN = 256, BK = 64, ROWB = 128;
  constexpr int ASTAGE = BM * ROWB;           // 40 KB
  constexpr int BSTAGE = BN * ROWB;           // 32 KB
  constexpr int WTM = 128, WTN = 128, NJ = 4;
  constexpr int BN_OUT = MODE == kGatedBf16 ? BN / 2 : BN;
  // bf16 outputs: the MFMAs compute the transposed tile (see the epilogue)
  constexpr bool kTr = MODE != kPlainF32;
  // weights stored [K][N] (a plain GEMM on the weights as they are, e.g. the input
  // gradient's dY W_down): a B stage is 64 weight rows (K) x 256 columns (N) of 512
  // bytes, 16-byte chunk c of row r in slot c ^ 4 (r & 7); fragments are read across
  // rows with ds_read_b64_tr_b16 (see read_b)
  constexpr bool kKN = MODE == kPlainKN;
  constexpr int NDA = BM / 32, NDB = BN / 32; // DMA instructions per wave per stage
  __shared__ __attribute__((aligned(1024))) uint4 lds[(2 * ASTAGE + 2 * BSTAGE) / 16];

  // ---- tiles ---------------------------------------------------------------------
  // Workgroups reach the XCDs round-robin (b % 8).  The row blocks (see build_schedule:
  // pairs of one expert's equal blocks, then lone blocks, each largest first) are dealt
  // to the XCDs in pairs of adjacent blocks in snake order (round r: XCDs 0..7, then
  // 7..0), so every XCD gets an even share and runs its largest blocks first; a pair's
  // n-tiles are consecutive slots of one XCD, so the two blocks of one expert stream
  // each weight tile side by side through that XCD's L2.  The expert GEMMs run persistent workgroups (one per CU; gridDim.x
  // = 8 x nwg): workgroup j of an XCD takes slots j, j + nwg, j + 2 nwg, ... and loads
  // the first stage of its next tile while it writes out the current one.  The
  // fp32-output mode (router logits, router backward) runs one workgroup per tile.
  constexpr bool PERSIST = MODE != kPlainF32;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int xcd = blockIdx.x % kXcds;
  const int nwg = PERSIST ? int(gridDim.x) / kXcds : 0;
  int slot = blockIdx.x / kXcds;
  const int nblocks = a.sched ? *a.sched_n : 0;
  // place of slot s of this XCD: schedule position pos, n-tile nt; valid if it has a block
  // slots walk pairs of adjacent schedule positions (pair q = round * 8 + the XCD's
  // snake place), the n-tiles of the pair's two blocks interleaved, so a busy expert's
  // consecutive blocks stream each weight tile side by side through one L2; an odd block
  // count leaves the last pair's second slots empty (skipped)
  auto place_of = [&](int s, int& pos_, int& nt_) __attribute__((always_inline)) {
    const int per = 2 * a.n_tiles;
    const int rp = s / per, rem = s - rp * per;
    nt_ = rem >> 1;
    const int q = rp * kXcds + ((rp & 1) ? kXcds - 1 - xcd : xcd);
    pos_ = 2 * q + (rem & 1);
    return pos_ < nblocks;
  };
  // slots past this one hold no block on any XCD
  const int slot_limit = ((nblocks + 1) / 2 + kXcds - 1) / kXcds * 2 * a.n_tiles;
  // tile of slot s: group g, rows m0 .. m0 + mvalid - 1, n-tile nt
  auto tile_of = [&](int s, int& g_, int& m0_, int& mvalid_, int& nt_) __attribute__((always_inline)) {
    int pos;
    if (a.sched) {
      if (!place_of(s, pos, nt_)) return false;
      const int4 e = a.sched[pos];
      g_ = e.x;
      m0_ = e.y;
      mvalid_ = e.z;
    } else {
      // one group of T rows, one workgroup per tile (not persistent): workgroup b takes
      // row block b / n_tiles, n-tile b % n_tiles, so any shape spreads over all XCDs
      // (a shape with fewer row blocks than XCDs included)
      const int b = int(blockIdx.x);
      const int mb = b / a.n_tiles;
      nt_ = b - mb * a.n_tiles;
      g_ = 0;
      m0_ = mb * BM;
      if (m0_ >= a.T) return false;
      mvalid_ = min(BM, a.T - m0_);
    }
    return true;
  };
  int g = 0, m0 = 0, mvalid = 0, nt = 0;
  if (a.sched) {
    // the first slot of this workgroup with a block
    while (slot < slot_limit && !tile_of(slot, g, m0, mvalid, nt)) slot += nwg;
    if (slot >= slot_limit) return;
  } else if (!tile_of(slot, g, m0, mvalid, nt)) return;
  int n0 = nt * BN_OUT;
  // split-K (router logits): this workgroup's K range, its own partial output slice
  const int kst0 = blockIdx.y * (a.k_chunk / BK);      // first stage
  const int K = a.k_chunk ? min(a.k_chunk, a.K - blockIdx.y * a.k_chunk) : a.K;
  const uint32_t row_bytes = uint32_t(a.K) * 2u;
  const uint32_t row_bytes_b = uint32_t(a.N) * 2u;      // [K][N] weights: one K row

  // ---- this wave's share of every stage: A rows 80 w.., B rows 64 w.. ---------------
  // B: the tile's first weight row (gated: of the gate and of the up half) is in the
  // buffer base, so the lane offsets hold for every tile; rows >= N read zero
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(a.A, uint32_t(a.a_rows) * row_bytes);
  const uint16_t* const bsel = MODE == kGatedBf16 && w >= 2 ? a.B1 : a.B0;
  auto rsrc_b_of = [&](int g_, int nt_) __attribute__((always_inline)) {
    const int nb = nt_ * BN_OUT;
    if constexpr (kKN)     // the tile's first column; K rows up to the split from B0
      return make_rsrc(a.B0 + size_t(g_) * a.b_stride + nb, (uint32_t(a.k_split) * uint32_t(a.N) - nb) * 2u);
    return make_rsrc(bsel + size_t(g_) * a.b_stride + size_t(nb) * a.K, uint32_t(a.N - nb) * row_bytes);
  };
  // [K][N] weights stacked along K: rows from k_split on come from B1
  auto rsrc_b1_of = [&](int g_, int nt_) __attribute__((always_inline)) {
    const int nb = nt_ * BN_OUT;
    const uint16_t* b1 = a.B1 ? a.B1 : a.B0;
    const uint32_t n1 = a.K > a.k_split ? (uint32_t(a.K - a.k_split) * uint32_t(a.N) - nb) * 2u : 0u;
    return make_rsrc(b1 + size_t(g_) * a.b_stride + nb, n1);
  };
  __amdgpu_buffer_rsrc_t rsrc_b = rsrc_b_of(g, nt);
  __amdgpu_buffer_rsrc_t rsrc_b1 = rsrc_b;
  if constexpr (kKN) rsrc_b1 = rsrc_b1_of(g, nt);
  uint32_t voff_a[NDA], voff_b[NDB];
  // A row offsets of a tile: routed rows (below TK) gather their token through
  // row_token; a tile of shared-expert rows maps to consecutive tokens
  int a_rows_valid = 0;                       // rows of the tile whose A offsets are set
  auto set_voff_a = [&](int m0_, int mvalid_) __attribute__((always_inline)) {
    a_rows_valid = mvalid_;
    const bool lookup = a.gather && m0_ < a.TK;
    const int base = !a.gather ? m0_ : (lookup ? 0 : (m0_ - a.TK) % a.T);
#pragma unroll
    for (int j = 0; j < NDA; ++j) {
      const int arow = (BM / 4) * w + 8 * j + (l >> 3);
      const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ (j & 1)) * 16u;
      uint32_t o = kOob;
      if (arow < mvalid_) {
        const int src = lookup ? a.row_token[m0_ + arow] : base + arow;
        o = uint32_t(src) * row_bytes + chunk;
      }
      voff_a[j] = o;
    }
  };
  set_voff_a(m0, mvalid);
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    if constexpr (kKN) {
      // K rows 16 w + 2 j + (l >> 5) of the stage, slot l & 31 of the row's 32
      const int kr = 16 * w + 2 * j + (l >> 5);
      const uint32_t chunk = uint32_t((l & 31) ^ (4 * (kr & 7))) * 16u;
      voff_b[j] = uint32_t(kr) * row_bytes_b + chunk;
      continue;
    }
    const int rw = 8 * j + (l >> 3);
    const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ (j & 1)) * 16u;
    // gated: B rows 0..127 are gate rows, 128..255 the matching up rows
    const int n = MODE == kGatedBf16 ? 64 * (w & 1) + rw : 64 * w + rw;
    voff_b[j] = uint32_t(n) * row_bytes + chunk;
  }
  // LDS: B buffers at [0, 64K), A buffers at [64K, 144K); stage k uses buffer k & 1
  constexpr uint32_t kAOff = 2 * BSTAGE;
  const uint32_t lds_base = uint32_t(uintptr_t(&lds[0]));
  const uint32_t wave_a = lds_base + kAOff + uint32_t(w) * (ASTAGE / 4);
  const uint32_t wave_b = lds_base + uint32_t(w) * (BSTAGE / 4);
  auto dma_a = [&](int ks, auto par_tag, auto j_tag) __attribute__((always_inline)) {
    constexpr int j = decltype(j_tag)::value, par = decltype(par_tag)::value;
    // 8-row groups wholly past the tile's rows are not loaded: their LDS rows keep
    // stale values, which reach only output rows that are never stored
    if ((BM / 4) * w + 8 * j < a_rows_valid)
      dma16(rsrc_a, voff_a[j], uint32_t(ks + kst0) * ROWB, wave_a + uint32_t(par * ASTAGE + j * 1024));
  };
  auto dma_b = [&](int ks, auto par_tag, auto j_tag) __attribute__((always_inline)) {
    constexpr int j = decltype(j_tag)::value, par = decltype(par_tag)::value;
    if constexpr (kKN) {
      const int kr0 = 64 * ks;                            // first K row of the stage
      const bool hi = kr0 >= a.k_split;
      dma16(hi ? rsrc_b1 : rsrc_b, voff_b[j], uint32_t(hi ? kr0 - a.k_split : kr0) * row_bytes_b,
            wave_b + uint32_t(par * BSTAGE + j * 1024));
      return;
    }
    dma16(rsrc_b, voff_b[j], uint32_t(ks + kst0) * ROWB, wave_b + uint32_t(par * BSTAGE + j * 1024));
  };

  // ---- fragment geometry: per-step lane bases; buffer and block offsets are immediates
  const int wm = w >> 1, wn = w & 1;
  // Set up again for every tile from a lane id the compiler cannot hoist: these values
  // then die with the K loop instead of staying live (and spilling) through the
  // epilogue of a persistent workgroup.
  uint32_t abase[4], bbase[4], xbase[4];
  // [K][N] weights: per lane, the byte of its first 8-byte transposed read in block j
  // (rows 8 (ll >> 5) + (ll & 15) / 4 of a 16-row K step) and of its second (4 rows on)
  uint32_t kn1[NJ], kn2[NJ];
  auto set_frag_bases = [&]() __attribute__((always_inline)) {
    int ll;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ll));
    if constexpr (kKN) {
      const int L = ll & 15, khalf = ll >> 5, nhalf = (ll >> 4) & 1;
      const int x1 = L >> 2, x2 = 4 + (L >> 2);          // row & 7 of the two reads
      const uint32_t row1 = uint32_t(8 * khalf + (L >> 2)) * 512u;
      const uint32_t inner = uint32_t(2 * nhalf + ((L & 3) >> 1)) * 16u + uint32_t(L & 1) * 8u;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        kn1[j] = row1 + uint32_t((4 * wn + j) ^ x1) * 64u + inner;
        kn2[j] = row1 + 2048u + uint32_t((4 * wn + j) ^ x2) * 64u + inner;
      }
    }
    const int lane_row = ll & 31;
    const int b_row0 = (MODE == kGatedBf16 ? wn * (WTN / 2) : wn * WTN) + lane_row;
    const int a_row = wm * WTM + lane_row;
    const int x_row = BMAIN + lane_row;                 // strip 1: + 32 rows
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const uint32_t sl = uint32_t((2 * s4 + (ll >> 5)) ^ (ll & 7) ^ ((ll >> 3) & 1)) * 16u;
      bbase[s4] = uint32_t(b_row0) * ROWB + sl;
      abase[s4] = kAOff + uint32_t(a_row) * ROWB + sl;
      xbase[s4] = kAOff + uint32_t(x_row) * ROWB + sl;
    }
  };
  // B block j of the wave: rows b_row0 + offset (gated: gate blocks, then up blocks)
  auto b_blk = [](int j) constexpr {
    return MODE == kGatedBf16 ? (j < NJ / 2 ? j * 32 : BN / 2 + (j - NJ / 2) * 32) : j * 32;
  };
  const int nk = K / BK;
  bool has_next = false;                     // next tile of this workgroup and its place
  int pos2 = 0, g2 = 0, m02 = 0, mv2 = 0, nt2 = 0, next_slot = 0;
  // the next tile's schedule entry, loaded at the start of a tile (a vector load: the
  // scalar-cache wait would land in the stage barriers) and read in its epilogue
  const __amdgpu_buffer_rsrc_t rsrc_sched = make_rsrc(a.sched, uint32_t(nblocks) * 16u);

  auto body = [&](auto niv_tag, auto x_tag, auto xw_tag) __attribute__((always_inline)) {
    constexpr int NIV = decltype(niv_tag)::value;
    constexpr int NX = decltype(x_tag)::value;     // extra strips with rows (0..2)
    constexpr int XW = decltype(xw_tag)::value;    // the wave's wm, for the extra blocks
    constexpr int NA = NIV + NX;                   // A fragments per K-step
    constexpr int NMS = NIV * NJ + 2 * NX;         // MFMAs per K-step
    // extra MFMA e: strip e / 2, B block xb(e) (gated: the gate block and its up block;
    // plain: two adjacent blocks, so the strip's outputs of a wave are 64 adjacent columns)
    constexpr auto xb = [](int e) constexpr {
      const int xh = (e >> 1) == 0 ? XW : 1 - XW;
      return MODE == kGatedBf16 ? xh + 2 * (e & 1) : 2 * xh + (e & 1);
    };
    constexpr int NRB = NA > 0 ? NJ : 0;           // B fragments per K-step (skipped if idle)
    f32x16_t acc[NIV > 0 ? NIV : 1][NJ];
    f32x16_t accx[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int i = 0; i < NIV; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }                                              // accx: defined by its first MFMA
    bf16x8_t fb[4][NJ];                            // B fragments of the four K-steps
    bf16x8_t fa[2][NA > 0 ? NA : 1];               // A fragments, double-buffered by step

    auto lds_read = [&](uint32_t byte) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                              reinterpret_cast<const char*>(lds) + byte));
    };
    // B fragment (step S4, block J) and A fragment (step S4, block I; I == NIV is the
    // extra strip) of the stage in buffer PAR
    auto read_b = [&](auto par_tag, auto s_tag, auto j_tag) __attribute__((always_inline)) {
      constexpr int par = decltype(par_tag)::value, s4 = decltype(s_tag)::value;
      constexpr int j = decltype(j_tag)::value;
      if constexpr (kKN) {
        // eight K values of one column (n = lane & 31) from two transposed reads: within
        // a group of 16 lanes, value q of lane i comes from element i & 3 of the 8 bytes
        // lane 4 q + i / 4 addresses
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const uint32_t off = uint32_t(par * BSTAGE + s4 * 16 * 512);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(reinterpret_cast<char*>(lds) + kn1[j] + off));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(reinterpret_cast<char*>(lds) + kn2[j] + off));
        fb[s4][j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        return;
      }
      fb[s4][j] = lds_read(bbase[s4] + uint32_t(par * BSTAGE + b_blk(j) * ROWB));
    };
    auto read_a = [&](auto par_tag, auto s_tag, auto i_tag) __attribute__((always_inline)) {
      constexpr int par = decltype(par_tag)::value, s4 = decltype(s_tag)::value;
      constexpr int i = decltype(i_tag)::value;
      if constexpr (i < NIV)
        fa[s4 & 1][i] = lds_read(abase[s4] + uint32_t(par * ASTAGE + i * 32 * ROWB));
      else
        fa[s4 & 1][i] = lds_read(xbase[s4] + uint32_t(par * ASTAGE + (i - NIV) * 32 * ROWB));
    };
    // FIRST: step 0 of stage 0, where the extra strip's accumulators start
    auto mfma_of = [&](auto s_tag, auto m_tag, auto first_tag) __attribute__((always_inline)) {
      constexpr int s4 = decltype(s_tag)::value, m = decltype(m_tag)::value;
      if constexpr (m < NIV * NJ) {
        constexpr int i = m / NJ, j = m % NJ;
        if constexpr (kTr)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s4][j], fa[s4 & 1][i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s4 & 1][i], fb[s4][j], acc[i][j], 0, 0, 0);
      } else {
        constexpr int e = m - NIV * NJ;
        const bf16x8_t& xa = fa[s4 & 1][NIV + (e >> 1)];
        const bf16x8_t& xbf = fb[s4][xb(e)];
        if constexpr (decltype(first_tag)::value)
          mfma_vgpr_first(accx[e], kTr ? xbf : xa, kTr ? xa : xbf);
        else
          mfma_vgpr(accx[e], kTr ? xbf : xa, kTr ? xa : xbf);
      }
    };
    auto none = [&](auto) __attribute__((always_inline)) {};
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    using T_ = std::true_type;
    using F_ = std::false_type;

    // One stage k in buffer PAR, entered right after the barrier that published it:
    //  R0  second half of stage k-1's step 3 (if PREV); reads of step 0; DMA A k+1 (if DA)
    //  R1  step 0; reads of B steps 1..3 and A step 1; then the barrier that frees B k
    //  R2  step 1; reads of A step 2; DMA B k+2 into B k's buffer (if DB)
    //  R3  step 2; reads of A step 3
    //  R4  first half of step 3; then publish stage k+1 (if PUB; VM loads may stay in flight)
    // VM < 0: the bound is chosen at run time (NDB when this stage's B loads went out,
    // else 0); with DB, the B loads of stage kb go out only when db_rt holds
    auto stage = [&](int k, auto par_tag, auto prev_tag, auto da_tag, auto db_tag, auto pub_tag,
                     auto vm_tag, int kb, bool db_rt) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_tag)::value;
      constexpr bool PREV = decltype(prev_tag)::value, DA = decltype(da_tag)::value;
      constexpr bool DB = decltype(db_tag)::value, PUB = decltype(pub_tag)::value;
      constexpr int VM = decltype(vm_tag)::value;
      using P = std::integral_constant<int, PAR>;
      using Q = std::integral_constant<int, 1 - PAR>;
      auto rd0 = [&](auto q_tag) __attribute__((always_inline)) {
        constexpr int q = decltype(q_tag)::value;
        if constexpr (q < NRB) read_b(P{}, S0{}, q_tag);
        else read_a(P{}, S0{}, std::integral_constant<int, q - NRB>{});
      };
      auto dma_a1 = [&](auto j_tag) __attribute__((always_inline)) { dma_a(k + 1, Q{}, j_tag); };
      interleave<NMS / 2, PREV ? NMS : NMS / 2, NRB + NA, DA ? NDA : 0>(
          [&](auto m) __attribute__((always_inline)) { mfma_of(S3{}, m, F_{}); }, rd0, dma_a1);
      auto rd1 = [&](auto q_tag) __attribute__((always_inline)) {
        constexpr int q = decltype(q_tag)::value;
        if constexpr (q < 3 * NRB)
          read_b(P{}, std::integral_constant<int, 1 + q / NJ>{}, std::integral_constant<int, q % NJ>{});
        else
          read_a(P{}, S1{}, std::integral_constant<int, q - 3 * NRB>{});
      };
      interleave<0, NMS, 3 * NRB + NA, 0>(
          [&](auto m) __attribute__((always_inline)) { mfma_of(S0{}, m, std::bool_constant<!PREV>{}); }, rd1, none);
      stage_barrier();                          // every wave holds its B k fragments
      auto rd2 = [&](auto q_tag) __attribute__((always_inline)) { read_a(P{}, S2{}, q_tag); };
      // B stage kb (k + 2, or a stage of the next tile) into the buffer stage k leaves
      auto dma_b2 = [&](auto j_tag) __attribute__((always_inline)) {
        if (db_rt) dma_b(kb, P{}, j_tag);
      };
      interleave<0, NMS, NA, DB ? NDB : 0>(
          [&](auto m) __attribute__((always_inline)) { mfma_of(S1{}, m, F_{}); }, rd2, dma_b2);
      auto rd3 = [&](auto q_tag) __attribute__((always_inline)) { read_a(P{}, S3{}, q_tag); };
      interleave<0, NMS, NA, 0>(
          [&](auto m) __attribute__((always_inline)) { mfma_of(S2{}, m, F_{}); }, rd3, none);
      interleave<0, NMS / 2, 0, 0>(
          [&](auto m) __attribute__((always_inline)) { mfma_of(S3{}, m, F_{}); }, none, none);
      if constexpr (PUB) {
        if constexpr (VM >= 0) {
          wait_vmcnt<VM>();
        } else {
          if (db_rt) wait_vmcnt<NDB>();
          else wait_vmcnt<0>();
        }
        stage_barrier();
      }
    };
    using V0 = std::integral_constant<int, 0>;
    using VB = std::integral_constant<int, NDB>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    // A 0, B 0 and B 1 are in flight (issued before the tile loop for the first tile,
    // during the previous tile's epilogue for the others)
    wait_vmcnt<0>();
    stage_barrier();
    i32x4_t next_e{};
    bool b_early = false;                    // the next tile's B 0 and B 1 already went out
    if constexpr (PERSIST) {
      if (has_next) next_e = __builtin_amdgcn_raw_buffer_load_b128(rsrc_sched, uint32_t(pos2) * 16u, 0, 0);
    }
    // nk = K / 64 is even (K is a multiple of 128)
    auto two_stages = [&]() __attribute__((always_inline)) {
      stage(0, P0{}, F_{}, T_{}, F_{}, T_{}, V0{}, 2, false);
      stage(1, P1{}, T_{}, F_{}, F_{}, F_{}, V0{}, 3, false);
    };
    auto k_loop = [&]() __attribute__((always_inline)) {
      stage(0, P0{}, F_{}, T_{}, T_{}, T_{}, VB{}, 2, true);
      stage(1, P1{}, T_{}, T_{}, T_{}, T_{}, VB{}, 3, true);
      for (int k = 2; k < nk - 2; k += 2) {
        stage(k, P0{}, T_{}, T_{}, T_{}, T_{}, VB{}, k + 2, true);
        stage(k + 1, P1{}, T_{}, T_{}, T_{}, T_{}, VB{}, k + 3, true);
      }
      // the next tile's B 0 and B 1 go out in the last two stages, into the buffers
      // those stages free (nk is even: the same parities), so their HBM latency hides
      // behind this tile's last MFMAs and epilogue; stage nk - 2 then publishes stage
      // nk - 1 with the next tile's B 0 still in flight
      if (PERSIST && has_next) {
        g2 = __builtin_amdgcn_readfirstlane(next_e[0]);
        m02 = __builtin_amdgcn_readfirstlane(next_e[1]);
        mv2 = __builtin_amdgcn_readfirstlane(next_e[2]);
        rsrc_b = rsrc_b_of(g2, nt2);
        if constexpr (kKN) rsrc_b1 = rsrc_b1_of(g2, nt2);
        b_early = true;
      }
      using VR = std::integral_constant<int, -1>;
      stage(nk - 2, P0{}, T_{}, T_{}, T_{}, T_{}, VR{}, 0, b_early);
      stage(nk - 1, P1{}, T_{}, F_{}, T_{}, F_{}, V0{}, 1, b_early);
    };
    if constexpr (SHORT_K) {
      two_stages();
    } else {
      k_loop();
    }
    interleave<NMS / 2, NMS, 0, 0>(
        [&](auto m) __attribute__((always_inline)) { mfma_of(S3{}, m, F_{}); }, none, none);

    // ---- epilogue -------------------------------------------------------------------
    // bf16 modes: the MFMAs compute the transposed tile (weight rows are the MFMA's
    // rows): value r of lane l of a 32 x 32 accumulator is output row l & 31 of its
    // block and column 8 (r >> 2) + 4 (l >> 5) + (r & 3), so each group of four values
    // is four adjacent columns of one row.
    if constexpr (NX > 0) mfma_vgpr_drain(accx);
    // lane id recomputed here: lane expressions shared with the prologue would otherwise
    // stay live (and spill) across the K loop
    const int le = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
    const int lr = le & 31, lh = le >> 5;
    if constexpr (MODE == kPlainF32) {
      // fp32 partials (not transposed: lane l holds column l & 31 of rows
      // 8 (r >> 2) + 4 (l >> 5) + (r & 3)), 128 contiguous bytes per row and store
      float* const cz = static_cast<float*>(a.C) + size_t(blockIdx.y) * a.c_split_stride;
      auto put_blk = [&](const f32x16_t& v, int rb, int col) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = rb + (r >> 2) * 8 + lh * 4 + (r & 3);
          if (rl < mvalid && col < a.N) cz[size_t(m0 + rl) * a.ldc + col] = v[r];
        }
      };
#pragma unroll
      for (int i = 0; i < NIV; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) put_blk(acc[i][j], wm * WTM + i * 32, n0 + wn * WTN + j * 32 + lr);
      static_for<0, 2 * NX>([&](auto e_tag) __attribute__((always_inline)) {
        constexpr int e = decltype(e_tag)::value;
        put_blk(accx[e], BMAIN + 32 * (e >> 1), n0 + wn * WTN + xb(e) * 32 + lr);
      });
    } else {
      stage_barrier();                          // every wave is done with this tile's LDS
      // the next tile's B 0 and B 1 now unless the last two stages sent them (K = 128);
      // its A 0 after the epilogue, which stages through A buffer 1
      if constexpr (PERSIST) {
        if (has_next && !b_early) {
          g2 = __builtin_amdgcn_readfirstlane(next_e[0]);
          m02 = __builtin_amdgcn_readfirstlane(next_e[1]);
          mv2 = __builtin_amdgcn_readfirstlane(next_e[2]);
          rsrc_b = rsrc_b_of(g2, nt2);
          if constexpr (kKN) rsrc_b1 = rsrc_b1_of(g2, nt2);
          static_for<0, NDB>([&](auto j) __attribute__((always_inline)) { dma_b(0, P0{}, j); });
          static_for<0, NDB>([&](auto j) __attribute__((always_inline)) { dma_b(1, P1{}, j); });
        }
      }
      // bf16 outputs go through LDS: each wave writes one 32-row block at a time into
      // its own 10 KB of A buffer 1 (8-byte writes of four adjacent columns), then reads
      // whole rows back 16 bytes per lane and stores them with full-line 16-byte buffer
      // stores.  A staging row of P bytes has P / 16 chunks; chunk c of row r sits in
      // slot c ^ ((r / (256 / P)) % (P / 16)): every 16-lane quarter of a read covers the
      // 64 banks once, a half-wave's writes hit each bank pair at most twice.  The store
      // buffer spans the tile's valid rows, so stores of rows past them are dropped by
      // the hardware's range check; columns past N get an offset past the range.
      char* const stg = reinterpret_cast<char*>(lds) + kAOff + ASTAGE + w * 10240;
      const uint32_t ldc2 = uint32_t(a.ldc) * 2u;
      const __amdgpu_buffer_rsrc_t rsrc_c =
          make_rsrc(static_cast<uint16_t*>(a.C) + size_t(m0) * a.ldc, uint32_t(mvalid) * ldc2);
      auto pack = [](float x0, float x1) __attribute__((always_inline)) { return pack_bf16x2(x0, x1); };
      // this lane's write slot base for pitch P: row lr, chunk 0, half lh
      auto wslot = [&](auto p_tag) __attribute__((always_inline)) {
        constexpr int P = decltype(p_tag)::value, CH = P / 16, RPB = 256 / P;
        return uint32_t(lr * P + (((lr / RPB) % CH) << 4) + (lh << 3));
      };
      auto put8 = [&](uint32_t slot8, int c, uint32_t lo, uint32_t hi) __attribute__((always_inline)) {
        *reinterpret_cast<uint2*>(stg + (slot8 ^ uint32_t(c << 4))) = make_uint2(lo, hi);
      };
      // the 32 staged rows of pitch P (P / 2 columns) to output rows m0 + rb + (0 .. 31),
      // columns from cb; rows past vrows are not stored
      auto drain = [&](auto p_tag, int rb, int vrows, int cb) __attribute__((always_inline)) {
        constexpr int P = decltype(p_tag)::value, CH = P / 16, RPB = 256 / P, RPI = 64 / CH;
        constexpr int NQ = 32 / RPI, QG = NQ < 4 ? NQ : 4;   // reads in flight per group
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int c = le % CH, col = cb + 8 * c;
        const uint32_t voff = col < a.N ? (uint32_t(rb + le / CH) * uint32_t(a.ldc) + uint32_t(col)) * 2u : kOob;
#pragma unroll
        for (int q0 = 0; q0 < NQ; q0 += QG) {
          if (q0 * RPI >= vrows) break;
          uint4 v[QG];
#pragma unroll
          for (int u = 0; u < QG; ++u) {
            const int r = (q0 + u) * RPI + le / CH;
            v[u] = *reinterpret_cast<const uint4*>(stg + r * P + ((c ^ ((r / RPB) % CH)) << 4));
          }
#pragma unroll
          for (int u = 0; u < QG; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v[u]), rsrc_c, voff,
                                                   uint32_t((q0 + u) * RPI) * ldc2, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      };
      const int wrows = mvalid - wm * WTM;                  // this wave's valid main rows
      // the strips go first: their VGPR accumulators are free before the next tile's A
      // offsets are computed
      if constexpr (MODE == kGatedBf16) {
        // strips: 32 columns per wave and strip (gate accx[2 st], up accx[2 st + 1])
        using PX = std::integral_constant<int, 64>;
        const uint32_t sx = wslot(PX{});
        static_for<0, NX>([&](auto st_tag) __attribute__((always_inline)) {
          constexpr int st = decltype(st_tag)::value;
          constexpr int xh = st == 0 ? XW : 1 - XW;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float hv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
              hv[t] = silu_fast(accx[2 * st][4 * g4 + t]) * accx[2 * st + 1][4 * g4 + t];
            put8(sx, g4, pack(hv[0], hv[1]), pack(hv[2], hv[3]));
          }
          drain(PX{}, BMAIN + 32 * st, mvalid - BMAIN - 32 * st, n0 + wn * (WTN / 2) + xh * 32);
        });
      } else {
        // strips: 64 adjacent columns per wave and strip (blocks xb(2 st), xb(2 st) + 1)
        using PX = std::integral_constant<int, 128>;
        const uint32_t sx = wslot(PX{});
        static_for<0, NX>([&](auto st_tag) __attribute__((always_inline)) {
          constexpr int st = decltype(st_tag)::value;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              put8(sx, 4 * h + g4, pack(accx[2 * st + h][4 * g4], accx[2 * st + h][4 * g4 + 1]),
                   pack(accx[2 * st + h][4 * g4 + 2], accx[2 * st + h][4 * g4 + 3]));
          drain(PX{}, BMAIN + 32 * st, mvalid - BMAIN - 32 * st, n0 + wn * WTN + xb(2 * st) * 32);
        });
      }
      if constexpr (MODE == kGatedBf16) {
        // h = silu(gate) * up: 64 columns per wave (gate blocks 0, 1 with up blocks 2, 3)
        using PW = std::integral_constant<int, 128>;
        const uint32_t sl = wslot(PW{});
#pragma unroll
        for (int i = 0; i < NIV; ++i) {
#pragma unroll
          for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              float hv[4];
#pragma unroll
              for (int t = 0; t < 4; ++t)
                hv[t] = silu_fast(acc[i][j][4 * g4 + t]) * acc[i][j + NJ / 2][4 * g4 + t];
              put8(sl, 4 * j + g4, pack(hv[0], hv[1]), pack(hv[2], hv[3]));
            }
          drain(PW{}, wm * WTM + i * 32, wrows - i * 32, n0 + wn * (WTN / 2));
        }
      } else {
        // 128 columns per wave
        using PW = std::integral_constant<int, 256>;
        const uint32_t sl = wslot(PW{});
#pragma unroll
        for (int i = 0; i < NIV; ++i) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              put8(sl, 4 * j + g4, pack(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1]),
                   pack(acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]));
          drain(PW{}, wm * WTM + i * 32, wrows - i * 32, n0 + wn * WTN);
        }
      }
      if constexpr (PERSIST) {
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // the first tile's stage 0 and B 1
  static_for<0, NDA>([&](auto j) __attribute__((always_inline)) { dma_a(0, I0{}, j); });
  static_for<0, NDB>([&](auto j) __attribute__((always_inline)) { dma_b(0, I0{}, j); });
  static_for<0, NDB>([&](auto j) __attribute__((always_inline)) { dma_b(1, I1{}, j); });
  for (;;) {
    set_frag_bases();
    if constexpr (PERSIST) {
      int s2 = slot + nwg;
      while (s2 < slot_limit && !place_of(s2, pos2, nt2)) s2 += nwg;
      has_next = s2 < slot_limit;
      next_slot = s2;
    }
    const int ni_valid = min(4, max(0, (min(mvalid, BMAIN) - wm * WTM + 31) >> 5));
    // rows 256..319 form two 32-row extra strips; every wave takes two 32-column blocks
    // of each strip that has rows (nx strips), so the four waves stay balanced
    const int nx = mvalid > BMAIN + 32 ? 2 : (mvalid > BMAIN ? 1 : 0);
    if (ni_valid > 2) {
      if (nx == 2) {
        if (wm == 0) body(std::integral_constant<int, 4>{}, I2{}, I0{});
        else body(std::integral_constant<int, 4>{}, I2{}, I1{});
      } else if (nx == 1) {
        if (wm == 0) body(std::integral_constant<int, 4>{}, I1{}, I0{});
        else body(std::integral_constant<int, 4>{}, I1{}, I1{});
      } else {
        body(std::integral_constant<int, 4>{}, I0{}, I0{});
      }
    } else if (ni_valid > 1) body(std::integral_constant<int, 2>{}, I0{}, I0{});
    else if (ni_valid > 0) body(std::integral_constant<int, 1>{}, I0{}, I0{});
    else body(std::integral_constant<int, 0>{}, I0{}, I0{});
    if (!has_next) break;
    // the next tile's A 0 (its B 0 and B 1 went out during the epilogue).  Computing
    // these offsets inside the epilogue makes the register allocator spill.
    set_voff_a(m02, mv2);
    static_for<0, NDA>([&](auto j) __attribute__((always_inline)) { dma_a(0, I0{}, j); });
    slot = next_slot;
    g = g2;
    m0 = m02;
    mvalid = mv2;
    nt = nt2;
    n0 = nt * BN_OUT;
  }
}

// Schedule of the expert GEMMs, one workgroup (G <= 512).  A group's rows split into
// c = ceil(rows / bm) blocks of at most bm rows, listed as {group, first row, rows};
// the output holds every row once, and the number of blocks.  A group gives c / 2
// pairs of consecutive blocks and, for odd c, a lone last block (the remainder); for
// even c the last pair splits the rows it covers evenly (the first block rounded up to
// 32 rows), so the two blocks of every pair do the same work.  The pairs come first,
// each on two adjacent positions from an even one, then the lone blocks; each kind by
// row count, largest first (a counting sort over 32-row classes, stable: units of one
// class keep the order of their groups, so the schedule is the same on every run).
// The bf16 expert GEMM runs the two blocks of positions 2q and 2q + 1 side by side on
// one XCD, so a pair streams each of its expert's weight tiles once through that L2.
__global__ __launch_bounds__(512) void build_schedule(const int32_t* __restrict__ offsets, int E,
                                                      int Ns, int T, int TK, int bm,
                                                      int4* __restrict__ sched,
                                                      int32_t* __restrict__ sched_n) {
  constexpr int kClasses = 64;              // 0..31 pairs, 32..63 lone blocks
  __shared__ int pre[512];
  __shared__ int cls_count[kClasses], cls_next[kClasses];
  const int t = threadIdx.x, G = E + Ns;
  int u = 0;
  if (t < G) {
    int r0, r1;
    group_rows(offsets, t, E, T, TK, r0, r1);
    const int c = ceil_div(r1 - r0, bm);
    u = c / 2 + (c & 1);
  }
  pre[t] = u;
  if (t < kClasses) cls_count[t] = 0;
  __syncthreads();
  for (int d = 1; d < 512; d <<= 1) {
    const int v = t >= d ? pre[t - d] : 0;
    __syncthreads();
    pre[t] += v;
    __syncthreads();
  }
  const int units = pre[G - 1];
  // unit id -> its group (the first g with pre[g] > id), first row, the rows of its
  // first block and of its second (0 for a lone block)
  struct Unit { int g, m0, rows0, rows1; };
  auto unit_of = [&](int id) {
    int lo = -1, hi = G - 1;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] > id) hi = mid; else lo = mid;
    }
    const int g = hi;
    const int j = id - (g > 0 ? pre[g - 1] : 0);
    int r0, r1;
    group_rows(offsets, g, E, T, TK, r0, r1);
    const int c = ceil_div(r1 - r0, bm);
    Unit un;
    un.g = g;
    if (j < c / 2) {
      un.m0 = r0 + 2 * j * bm;
      if ((c & 1) || j < c / 2 - 1) {        // two whole blocks
        un.rows0 = bm;
        un.rows1 = bm;
      } else {                                // the last pair: bm < rest <= 2 bm, split
        const int rest = r1 - un.m0;
        un.rows0 = min(bm, ((rest + 1) / 2 + 31) & ~31);
        un.rows1 = rest - un.rows0;
      }
    } else {                                  // the remainder of an odd count
      un.m0 = r0 + (c - 1) * bm;
      un.rows0 = r1 - un.m0;
      un.rows1 = 0;
    }
    return un;
  };
  auto cls_of = [&](const Unit& un) {
    return un.rows1 > 0 ? min(31, (2 * bm - un.rows0 - un.rows1) >> 5)
                        : 32 + min(31, (bm - un.rows0) >> 5);
  };
  // positions per unit of class k
  auto width = [](int k) { return k < 32 ? 2 : 1; };
  for (int id = t; id < units; id += 512) atomicAdd(&cls_count[cls_of(unit_of(id))], 1);
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int k = 0; k < kClasses; ++k) {
      cls_next[k] = acc;
      acc += width(k) * cls_count[k];
    }
    *sched_n = acc;
  }
  __syncthreads();
  // stable placement: 512 units at a time, each unit's rank among the same-class
  // units of its wave from ballots, the waves' per-class counts added in wave order
  __shared__ int wcount[8][kClasses];
  const int lane = t & 63, wv = t >> 6;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  for (int base = 0; base < units; base += 512) {
    const int id = base + t;
    const bool valid = id < units;
    Unit un{0, 0, 0, 0};
    int cl = -1;
    if (valid) {
      un = unit_of(id);
      cl = cls_of(un);
    }
    wcount[wv][lane] = 0;                   // kClasses == 64: one entry per lane
    __syncthreads();
    uint64_t left = __ballot(valid);
    int rank = 0;
    while (left) {
      const int leader = __ffsll((unsigned long long)left) - 1;
      const int lc = __shfl(cl, leader);
      const uint64_t same = __ballot(valid && cl == lc);
      if (valid && cl == lc) rank = __popcll(same & below);
      if (lane == leader) wcount[wv][lc] = __popcll(same);
      left &= ~same;
    }
    __syncthreads();
    if (valid) {
      int n = rank;
      for (int w2 = 0; w2 < wv; ++w2) n += wcount[w2][cl];
      const int pos = cls_next[cl] + width(cl) * n;
      sched[pos] = make_int4(un.g, un.m0, un.rows0, 0);
      if (un.rows1 > 0) sched[pos + 1] = make_int4(un.g, un.m0 + un.rows0, un.rows1, 0);
    }
    __syncthreads();
    if (t < kClasses) {
      int n = 0;
      for (int w2 = 0; w2 < 8; ++w2) n += wcount[w2][t];
      cls_next[t] += width(t) * n;
    }
    __syncthreads();
  }
}

// ---- fp32 path (small fp32 workloads): one thread per output element ---------
__device__ __forceinline__ int group_of_row(const int32_t* offsets, int r, int E, int T, int TK) {
  if (r >= TK) return E + (r - TK) / T;
  int lo = 0, hi = E;                     // largest e with offsets[e] <= r
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gemm1_f32(const float* __restrict__ x,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ row_token,
                                                 const float* __restrict__ wg,
                                                 const float* __restrict__ wu, int rows, int E,
                                                 int T, int TK, int H, int I,
                                                 float* __restrict__ h) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * I) return;
  const int r = i / I, n = i % I;
  const int e = group_of_row(offsets, r, E, T, TK);
  const float* xr = x + size_t(row_token_of(row_token, r, T, TK)) * H;
  const float* g = wg + (size_t(e) * I + n) * H;
  const float* u = wu + (size_t(e) * I + n) * H;
  float ag = 0.f, au = 0.f;
  for (int k = 0; k < H; ++k) {
    ag = fmaf(xr[k], g[k], ag);
    au = fmaf(xr[k], u[k], au);
  }
  h[i] = ag / (1.0f + expf(-ag)) * au;
}

__global__ __launch_bounds__(256) void gemm2_f32(const float* __restrict__ h,
                                                 const int32_t* __restrict__ offsets,
                                                 const float* __restrict__ wd, int rows, int E,
                                                 int T, int TK, int H, int I,
                                                 float* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * H) return;
  const int r = i / H, n = i % H;
  const int e = group_of_row(offsets, r, E, T, TK);
  const float* hr = h + size_t(r) * I;
  const float* d = wd + (size_t(e) * H + n) * I;
  float acc = 0.f;
  for (int k = 0; k < I; ++k) acc = fmaf(hr[k], d[k], acc);
  y[i] = acc;
}

// ---- launch configuration ---------------------------------------------------


hipError_t launch_gemm_router_bf16(const moe_config& c, const uint16_t* x, const uint16_t* w,
                                   float* z, hipStream_t s) {
  // one group of T rows, blocks of kExpertBM rows x all E columns, split-K over
  // router_splits(c) K ranges into fp32 partials [splits, T, E] (summed in order by the
  // selection kernel)
  GemmArgs a{};
  a.A = x;
  a.B0 = w;
  a.b_stride = 0;
  a.C = z;
  a.ldc = c.num_experts;
  a.N = c.num_experts;
  a.K = c.hidden;
  a.T = c.num_tokens;
  a.n_tiles = ceil_div(c.num_experts, 256);
  a.a_rows = c.num_tokens;
  a.k_chunk = router_k_chunk(c);
  a.c_split_stride = 1LL * c.num_tokens * c.num_experts;
  const dim3 grid(ceil_div(c.num_tokens, kExpertBM) * a.n_tiles, router_splits(c));
  if (c.hidden == 128) hipLaunchKernelGGL((grouped_gemm_dma<kPlainF32, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((grouped_gemm_dma<kPlainF32, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& a, int splits, hipStream_t s) {
  const int kc = a.k_chunk ? a.k_chunk : a.K;
  const int last = a.K - (splits - 1) * kc;
  if (a.K % 128 || kc % 128 || splits < 1 || (splits > 1 && !a.k_chunk) ||
      (kc == 128 ? last != 128 : (kc < 256 || last < 256 || last > kc)))
    return hipErrorInvalidValue;
  const dim3 grid(ceil_div(a.T, kExpertBM) * a.n_tiles, splits);
  if (kc == 128) hipLaunchKernelGGL((grouped_gemm_dma<kPlainF32, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((grouped_gemm_dma<kPlainF32, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_build_schedule(const moe_config& c, const int32_t* offsets, int bm, int4* sched,
                                 int32_t* sched_n, hipStream_t s) {
  const int T = c.num_tokens, E = c.num_experts, Ns = c.num_shared;
  hipLaunchKernelGGL(build_schedule, dim3(1), dim3(512), 0, s, offsets, E, Ns, T, T * c.top_k, bm,
                     sched, sched_n);
  return hipGetLastError();
}

// Workgroups resident at once (one per CU: the expert GEMMs take 144 KB of LDS), a
// multiple of the XCD count.  Cached per device; concurrent first calls store the same
// value.
static int resident_workgroups() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const bool cacheable = dev >= 0 && dev < 64;
  if (cacheable) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  n = n / kXcds * kXcds;
  if (n < kXcds) n = kXcds;
  if (cacheable) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_grouped_ffn(const moe_config& c, const void* x, const int32_t* offsets,
                              const int32_t* row_token, const moe_expert_weights& w,
                              void* y_rows, const Workspace& ws, hipStream_t s) {
  const int T = c.num_tokens, E = c.num_experts, Ns = c.num_shared;
  const int TK = T * c.top_k, rows = TK + T * Ns;
  const int H = c.hidden, I = c.inter;
  if (c.w_dtype == MOE_F32) {
    hipLaunchKernelGGL(gemm1_f32, dim3(ceil_div(rows * I, 256)), dim3(256), 0, s,
                       static_cast<const float*>(x), offsets, row_token,
                       static_cast<const float*>(w.w_gate), static_cast<const float*>(w.w_up),
                       rows, E, T, TK, H, I, static_cast<float*>(ws.h));
    hipLaunchKernelGGL(gemm2_f32, dim3(ceil_div(rows * H, 256)), dim3(256), 0, s,
                       static_cast<const float*>(ws.h), offsets,
                       static_cast<const float*>(w.w_down), rows, E, T, TK, H, I,
                       static_cast<float*>(y_rows));
    return hipGetLastError();
  }
  if (is_fp8(c.w_dtype))
    return launch_grouped_ffn_fp8(c, x, offsets, row_token, w, y_rows, ws, s);
  hipError_t err = launch_build_schedule(c, offsets, kExpertBM, ws.sched, ws.sched_n, s);
  if (err != hipSuccess) return err;
  // persistent workgroups: 8 x nwg, nwg per XCD, each XCD holding up to rounds x n_tiles
  // slots (rounds = the XCD's share of the row blocks)
  const int rounds = ceil_div(expert_row_blocks_upper(c, kExpertBM), kXcds);
  auto persistent_grid = [&](int n_tiles) {
    const int nwg = std::min(resident_workgroups() / kXcds, rounds * n_tiles);
    return dim3(unsigned(nwg * kXcds));
  };
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(x);
  a.row_token = row_token;
  a.sched = ws.sched;
  a.sched_n = ws.sched_n;
  a.B0 = static_cast<const uint16_t*>(w.w_gate);
  a.B1 = static_cast<const uint16_t*>(w.w_up);
  a.b_stride = 1LL * I * H;
  a.C = ws.h;
  a.ldc = I;
  a.N = I;
  a.K = H;
  a.T = T;
  a.TK = TK;
  a.n_tiles = ceil_div(I, 128);
  a.gather = 1;
  a.a_rows = T;
  const dim3 grid1 = persistent_grid(a.n_tiles);
  if (H == 128) hipLaunchKernelGGL((grouped_gemm_dma<kGatedBf16, true>), grid1, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((grouped_gemm_dma<kGatedBf16, false>), grid1, dim3(256), 0, s, a);
  GemmArgs d = a;
  d.A = static_cast<const uint16_t*>(ws.h);
  d.row_token = nullptr;
  d.gather = 0;
  d.a_rows = rows;
  d.B0 = static_cast<const uint16_t*>(w.w_down);
  d.B1 = nullptr;
  d.b_stride = 1LL * H * I;
  d.C = y_rows;
  d.ldc = H;
  d.N = H;
  d.K = I;
  d.n_tiles = ceil_div(H, 256);
  const dim3 grid2 = persistent_grid(d.n_tiles);
  if (I == 128) hipLaunchKernelGGL((grouped_gemm_dma<kPlainBf16, true>), grid2, dim3(256), 0, s, d);
  else hipLaunchKernelGGL((grouped_gemm_dma<kPlainBf16, false>), grid2, dim3(256), 0, s, d);
  return hipGetLastError();
}

// A plain grouped GEMM C[r] = A[r] B_e^T over the row blocks of a.sched (built by
// launch_build_schedule with kExpertBM-row blocks): the expert backward's products.
hipError_t launch_grouped_plain_bf16(const moe_config& c, const GemmArgs& a, hipStream_t s) {
  const int rounds = ceil_div(expert_row_blocks_upper(c, kExpertBM), kXcds);
  const int nwg = std::min(resident_workgroups() / kXcds, rounds * a.n_tiles);
  const dim3 grid(unsigned(nwg * kXcds));
  if (a.K == 128) hipLaunchKernelGGL((grouped_gemm_dma<kPlainBf16, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((grouped_gemm_dma<kPlainBf16, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// The same product on weights stored [K][N] per expert, read as they are: B0 holds K
// rows 0 .. k_split - 1, B1 (if K > k_split) rows k_split .. K - 1, b_stride elements
// per expert in each.  N a multiple of 8 (a tile's columns past N load whatever follows
// in the row, or zeros past the buffer; they feed only output columns that are not
// stored), K a multiple of 128, k_split of 64.
hipError_t launch_grouped_kn_bf16(const moe_config& c, const GemmArgs& a, hipStream_t s) {
  if (a.N % 8 || a.K % 128 || a.k_split % 64 || a.k_split <= 0 || a.k_split > a.K ||
      (a.k_split < a.K && !a.B1))
    return hipErrorInvalidValue;
  const int rounds = ceil_div(expert_row_blocks_upper(c, kExpertBM), kXcds);
  const int nwg = std::min(resident_workgroups() / kXcds, rounds * a.n_tiles);
  const dim3 grid(unsigned(nwg * kXcds));
  if (a.K == 128) hipLaunchKernelGGL((grouped_gemm_dma<kPlainKN, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((grouped_gemm_dma<kPlainKN, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
