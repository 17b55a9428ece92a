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
// Expert GEMMs use grouped_gemm_big (below); the router logits use the simpler
// 128 x 128 grouped_gemm_bf16 (v_mfma_f32_16x16x32_bf16, padded LDS, one slice of
// prefetch).  In both, GEMM1's B tile stacks BN/2 gate rows over the matching BN/2
// up rows and every wave owns the same columns of both halves, so the SwiGLU
// epilogue runs in registers; accumulation is fp32.
// Tile order: (expert, n-tile, m-tile) with m innermost, and the linear
// workgroup id is remapped so that each of the 8 XCDs (workgroups are dispatched
// round-robin over them) walks one contiguous stretch of that order: m-tiles of
// one weight tile, and n-tiles of one expert's rows, then share the XCD's L2.

#include <type_traits>

#include "gemm_common.h"

namespace moe {



template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_bf16(GemmArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 64;
  constexpr int LD = BK + 8;                  // padded LDS row pitch (bf16 elements)
  constexpr int WTM = BM / WM, WTN = BN / WN; // wave tile: rows x B-rows
  constexpr int NI = WTM / 16, NJ = WTN / 16;
  constexpr int CA = BM * (BK / 8) / NT;      // 16-byte chunks per thread per slice
  constexpr int CB = BN * (BK / 8) / NT;
  constexpr int BN_OUT = MODE == kGatedBf16 ? BN / 2 : BN;
  static_assert(CA * NT == BM * (BK / 8) && CB * NT == BN * (BK / 8), "tile/threads");
  static_assert(MODE != kGatedBf16 || NJ % 2 == 0, "gated tiles pair gate/up blocks");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LD];

  // ---- tile decode --------------------------------------------------------
  const int total_m = a.tile_off ? a.tile_off[a.G] : ceil_div(a.T, BM);
  const int total = total_m * a.n_tiles;
  const int b = blockIdx.x;
  if (b >= total) return;
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;

  int g, nt, mt, r0, r1;
  if (a.tile_off) {
    int lo = 0, hi = a.G;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (a.tile_off[mid] * a.n_tiles <= logical) lo = mid; else hi = mid;
    }
    g = lo;
    const int mtiles = a.tile_off[g + 1] - a.tile_off[g];
    const int local = logical - a.tile_off[g] * a.n_tiles;
    nt = local / mtiles;
    mt = local % mtiles;
    group_rows(a.offsets, g, a.E, a.T, a.TK, r0, r1);
  } else {
    g = 0;
    nt = logical / total_m;
    mt = logical % total_m;
    r0 = 0;
    r1 = a.T;
  }
  const int m0 = r0 + mt * BM;
  const int mvalid = min(BM, r1 - m0);
  const int n0 = nt * BN_OUT;

  const int tid = threadIdx.x;
  const int K = a.K;
  // split-K (router): this block sums K range [kbeg, kbeg + klen) into partial ks
  const int ks = blockIdx.y;
  const int kbeg = ks * a.k_chunk;
  const int klen = min(a.k_chunk, K - kbeg);

  // ---- per-thread global source pointers ----------------------------------
  const uint16_t* pa[CA];
  const uint16_t* pb[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + i * NT;
    const int row = min(c >> 3, mvalid - 1);      // padding rows re-read the last valid row
    const int r = m0 + row;
    const int src = a.gather ? row_token_of(a.row_token, r, a.T, a.TK) : r;
    pa[i] = a.A + size_t(src) * K + kbeg + (c & 7) * 8;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + i * NT;
    const int brow = c >> 3;
    const uint16_t* base = a.B0;
    int n = n0 + brow;
    if (MODE == kGatedBf16 && brow >= BN / 2) {
      base = a.B1;
      n = n0 + brow - BN / 2;
    }
    n = min(n, a.N - 1);
    pb[i] = base + size_t(g) * a.b_stride + size_t(n) * K + kbeg + (c & 7) * 8;
  }

  uint4 ra[CA], rb[CB];
  auto load_slice = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const uint4*>(pa[i] + k0);
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[i] = *reinterpret_cast<const uint4*>(pb[i] + k0);
  };
  auto store_slice = [&]() {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&As[(c >> 3) * LD + (c & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&Bs[(c >> 3) * LD + (c & 7) * 8]) = rb[i];
    }
  };

  const int w = tid >> 6, l = tid & 63;
  const int wm = w / WN, wn = w % WN;
  int brow0[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (MODE == kGatedBf16) {
      brow0[j] = j < NJ / 2 ? wn * (WTN / 2) + j * 16 : BN / 2 + wn * (WTN / 2) + (j - NJ / 2) * 16;
    } else {
      brow0[j] = wn * WTN + j * 16;
    }
  }

  f32x4_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = klen / BK;
  load_slice(0);
  for (int kt = 0; kt < nk; ++kt) {
    store_slice();
    __syncthreads();
    if (kt + 1 < nk) load_slice((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t af[NI], bfr[NJ];
      const int koff = ks * 32 + (l >> 4) * 8;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * WTM + i * 16 + (l & 15)) * LD + koff]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[(brow0[j] + (l & 15)) * LD + koff]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue: lane l holds rows (l/16)*4 + q, column l%16 of each 16x16 block
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rl = wm * WTM + i * 16 + (l >> 4) * 4 + q;
      if (rl >= mvalid) continue;
      const size_t row = size_t(m0 + rl);
      if (MODE == kGatedBf16) {
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
          const int col = n0 + wn * (WTN / 2) + j * 16 + (l & 15);
          const float gt = acc[i][j][q], up = acc[i][j + NJ / 2][q];
          const float hv = gt / (1.0f + expf(-gt)) * up;
          if (col < a.N) static_cast<uint16_t*>(a.C)[row * a.ldc + col] = f32_to_bf16_bits(hv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = n0 + wn * WTN + j * 16 + (l & 15);
          if (col >= a.N) continue;
          if (MODE == kPlainF32)
            static_cast<float*>(a.C)[ks * a.c_split_stride + row * a.ldc + col] = acc[i][j][q];
          else
            static_cast<uint16_t*>(a.C)[row * a.ldc + col] = f32_to_bf16_bits(acc[i][j][q]);
        }
      }
    }
  }
}

// ---- large-tile kernel for the expert GEMMs ---------------------------------
// A workgroup of 4 waves owns a BM x BN tile (256 x 256: an average expert at
// T = 8192 fits one m-tile); each wave owns a 128 x 128 sub-tile as 4 x 4 blocks
// of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane).  K advances in
// 64-wide slices through two LDS buffers; global reads are buffer loads (one
// descriptor per operand, per expert for the weights, K position in the scalar
// offset; rows past the tile or past N read as zero through the range check).
// Software pipeline per slice (four 16-wide K steps): each step's MFMAs run while
// the next step's fragments are read from LDS; after step 0 the next slice moves
// from registers into the other LDS buffer, one 16-byte write and one buffer load
// per MFMA, so the loads of slice k+2 have about four steps to land; the single
// barrier sits between steps 2 and 3 and orders LDS only (a full __syncthreads
// would drain the in-flight loads).  Scheduling-group hints keep the compiler
// from collapsing that order.  The number of valid 32-row blocks per wave (0, 1,
// 2 or 4) is a compile-time variant picked once per wave, so short tail tiles of
// an expert skip MFMA work without branches in the K loop.
// LDS rows are 8 16-byte chunks; chunk c of row r is stored in slot
// c ^ (r & 7) ^ ((r >> 3) & 1), which keeps the row-wise 128-byte stores and the
// 32-row fragment reads free of bank conflicts in every 8- or 16-lane group.
// Instruction-order hints for the scheduler (one ordered chain per region):
// masks 0x008 MFMA, 0x020 VMEM read, 0x100 DS read, 0x200 DS write.
template <int MASK, int SIZE>
__device__ __forceinline__ void sched_group() {
  if constexpr (SIZE > 0) __builtin_amdgcn_sched_group_barrier(MASK, SIZE, 0);
}
// NR fragment reads, then NM MFMAs of which the first NX are each followed by one
// LDS write and one buffer load (the register-to-LDS move of the next slice)
template <int NR, int NM, int NX>
__device__ __forceinline__ void sched_step() {
  if constexpr (NX == 0) {
    sched_group<0x100, NR>();
    sched_group<0x008, NM>();
  } else {
    sched_group<0x100, NR>();
    sched_group<0x008, 1>();
    sched_group<0x200, 1>();
    sched_group<0x020, 1>();
    sched_step<0, NM - 1, NX - 1>();
  }
}

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_big(GemmArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int CA = BM * 8 / NT, CB = BN * 8 / NT;   // 16-byte chunks per thread per slice
  constexpr int ROWS = BM + BN;
  constexpr int BN_OUT = MODE == kGatedBf16 ? BN / 2 : BN;
  static_assert(CA * NT == BM * 8 && CB * NT == BN * 8, "tile/threads");
  static_assert((NT / 8) % 16 == 0 && BM % 16 == 0, "store slots repeat every NT/8 rows");
  static_assert(MODE != kGatedBf16 || ((WTN / 32) % 2 == 0 && CB % 2 == 0), "gated tiles pair gate/up");
  __shared__ uint4 lds[2][ROWS * 8];

  // ---- tile decode ------------------------------------------------------------
  const int total_m = a.tile_off[a.G];
  const int total = total_m * a.n_tiles;
  const int b = blockIdx.x;
  if (b >= total) return;
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
  int lo = 0, hi = a.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tile_off[mid] * a.n_tiles <= logical) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mtiles = a.tile_off[g + 1] - a.tile_off[g];
  const int local = logical - a.tile_off[g] * a.n_tiles;
  const int nt = local / mtiles, mt = local % mtiles;
  int r0, r1;
  group_rows(a.offsets, g, a.E, a.T, a.TK, r0, r1);
  const int m0 = r0 + mt * BM;
  const int mvalid = min(BM, r1 - m0);
  const int n0 = nt * BN_OUT;
  const int tid = threadIdx.x;
  const int K = a.K;
  const uint32_t row_bytes = uint32_t(K) * 2u;

  // ---- buffer descriptors and per-lane offsets ----------------------------------
  const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(a.A, uint32_t(a.a_rows) * row_bytes);
  const uint32_t b_bytes = uint32_t(a.N) * row_bytes;
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(a.B0 + size_t(g) * a.b_stride, b_bytes);
  const __amdgpu_buffer_rsrc_t rb1 =
      MODE == kGatedBf16 ? make_rsrc(a.B1 + size_t(g) * a.b_stride, b_bytes) : rb0;
  const int trow = tid >> 3, kc0 = tid & 7;
  uint32_t oa[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int row = trow + i * (NT / 8);
    uint32_t o = kOob;
    if (row < mvalid) {
      const int r = m0 + row;
      const int src = a.gather ? row_token_of(a.row_token, r, a.T, a.TK) : r;
      o = uint32_t(src) * row_bytes + kc0 * 16;
    }
    oa[i] = o;
  }
  // B chunk i covers weight row n0 + trow + i*NT/8 (gated: the second half is up rows)
  constexpr int CBH = MODE == kGatedBf16 ? CB / 2 : CB;
  const uint32_t ob = uint32_t(n0 + trow) * row_bytes + kc0 * 16;
  const uint32_t ob_step = uint32_t(NT / 8) * row_bytes;
  const int st_base = trow * 8 + lds_slot(trow, kc0);       // + i*NT for chunk i

  uint4 ra[CA], rb[CB];
  auto load_slice = [&](int k0) __attribute__((always_inline)) {
    const int kb = k0 * 2;
#pragma unroll
    for (int i = 0; i < CA; ++i)
      ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra_src, oa[i], kb, 0));
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int ih = i < CBH ? i : i - CBH;
      rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          i < CBH ? rb0 : rb1, ob + uint32_t(ih) * ob_step, kb, 0));
    }
  };
  auto store_slice = [&](uint4* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CA; ++i) buf[st_base + i * NT] = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) buf[BM * 8 + st_base + i * NT] = rb[i];
  };

  // ---- wave geometry (wave index made scalar so tile-shape branches are uniform) --
  // MFMA 32x32x16: lane l supplies row/column l%32 at K chunk (l/32) of each 16-wide
  // K step, and holds output rows (r/4)*8 + (l/32)*4 + r%4, column l%32, r < 16.
  constexpr int NI32 = WTM / 32, NJ32 = WTN / 32;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int wm = w / WN, wn = w % WN;
  const int ni_valid = min(NI32, max(0, (mvalid - wm * WTM + 31) >> 5));
  const int a_base = (wm * WTM + (l & 31)) * 8;
  int b_row0[NJ32];
#pragma unroll
  for (int j = 0; j < NJ32; ++j) {
    int r;
    if (MODE == kGatedBf16)
      r = j < NJ32 / 2 ? wn * (WTN / 2) + j * 32 : BN / 2 + wn * (WTN / 2) + (j - NJ32 / 2) * 32;
    else
      r = wn * WTN + j * 32;
    b_row0[j] = (BM + r + (l & 31)) * 8;
  }
  const int nk = K / BK;   // even: K is a multiple of 128

  // The wave's whole tile computation for NIV valid 32-row blocks (0, 1, 2 or 4),
  // so the K loop itself has no branches: short tiles skip MFMA work per wave and
  // waves without valid rows only load, store and synchronise.
  auto body = [&](auto niv_tag) __attribute__((always_inline)) {
    constexpr int NIV = decltype(niv_tag)::value;
    f32x16_t acc[NIV > 0 ? NIV : 1][NJ32];
#pragma unroll
    for (int i = 0; i < NIV; ++i)
#pragma unroll
      for (int j = 0; j < NJ32; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Fragments of one 16-wide K step (s = 0..3 within the 64-wide slice).  The
    // fragment rows are 32-aligned + l%32, so the LDS slot depends only on l and s.
    struct Frag {
      bf16x8_t b[NJ32];
      bf16x8_t a[NIV > 0 ? NIV : 1];
    };
    auto read_frags = [&](Frag& f, const uint4* buf, int s) __attribute__((always_inline)) {
      if constexpr (NIV > 0) {
        const int sl = lds_slot(l & 31, s * 2 + (l >> 5));
#pragma unroll
        for (int j = 0; j < NJ32; ++j) f.b[j] = __builtin_bit_cast(bf16x8_t, buf[b_row0[j] + sl]);
#pragma unroll
        for (int i = 0; i < NIV; ++i) f.a[i] = __builtin_bit_cast(bf16x8_t, buf[a_base + i * 256 + sl]);
      }
    };
    auto mfmas = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NIV; ++i)
#pragma unroll
        for (int j = 0; j < NJ32; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };
    // Slice kt from `cur` (its step-0 fragments already in f0).  Software pipeline:
    // every step's MFMAs run while the next step's fragments are read; after step 0
    // slice kt+1 moves from registers into `nxt` and the loads of slice kt+2 are
    // issued (about four steps before they are needed); the one barrier sits between
    // steps 2 and 3, so step 3's MFMAs cover the first reads of the next slice.
    Frag f0, f1;
    auto slice = [&](const uint4* cur, uint4* nxt, int kt, auto st, auto ld, auto next,
                     auto prev) __attribute__((always_inline)) {
      constexpr int NR = NIV > 0 ? NIV + NJ32 : 0, NM = NIV * NJ32;
      constexpr int NX = decltype(st)::value && decltype(ld)::value ? (CA + CB < NM ? CA + CB : NM) : 0;
      read_frags(f1, cur, 1);
      mfmas(f0);
      if constexpr (decltype(st)::value) store_slice(nxt);
      if constexpr (decltype(ld)::value) load_slice((kt + 2) * BK);
      read_frags(f0, cur, 2);
      mfmas(f1);
      read_frags(f1, cur, 3);
      mfmas(f0);
      // region order: this slice's step-0 reads with the previous slice's step-3
      // MFMAs (none after the prologue), then steps 0..2, each preceded by the reads
      // of the step after it
      if constexpr (decltype(prev)::value) sched_step<NR, NM, 0>();
      else sched_step<NR, 0, 0>();
      sched_step<NR, NM, NX>();
      sched_step<NR, NM, 0>();
      sched_step<NR, NM, 0>();
      lds_barrier();
      if constexpr (decltype(next)::value) read_frags(f0, nxt, 0);
      mfmas(f1);
    };
    using yes = std::true_type;
    using no = std::false_type;

    load_slice(0);
    store_slice(lds[0]);
    load_slice(BK);
    lds_barrier();
    read_frags(f0, lds[0], 0);
    // slice kt reads lds[kt & 1]; slices 0 .. nk-3 also store slice kt+1 and load
    // slice kt+2, slice nk-2 only stores, slice nk-1 does neither (nk is even)
    if (nk == 2) {
      slice(lds[0], lds[1], 0, yes{}, no{}, yes{}, no{});
      slice(lds[1], lds[0], 1, no{}, no{}, no{}, yes{});
    } else {
      slice(lds[0], lds[1], 0, yes{}, yes{}, yes{}, no{});
      int kt = 1;
      for (; kt + 4 <= nk; kt += 2) {       // pairs of full slices (odd, even)
        slice(lds[1], lds[0], kt, yes{}, yes{}, yes{}, yes{});
        slice(lds[0], lds[1], kt + 1, yes{}, yes{}, yes{}, yes{});
      }
      slice(lds[1], lds[0], kt, yes{}, yes{}, yes{}, yes{});           // kt == nk-3
      slice(lds[0], lds[1], kt + 1, yes{}, no{}, yes{}, yes{});        // nk-2
      slice(lds[1], lds[0], kt + 2, no{}, no{}, no{}, yes{});          // nk-1
    }

    // ---- epilogue ---------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * WTM + i * 32 + (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
        if (rl >= mvalid) continue;
        const size_t row = size_t(m0 + rl);
        if (MODE == kGatedBf16) {
#pragma unroll
          for (int j = 0; j < NJ32 / 2; ++j) {
            const int col = n0 + wn * (WTN / 2) + j * 32 + (l & 31);
            const float hv = silu_fast(acc[i][j][r]) * acc[i][j + NJ32 / 2][r];
            if (col < a.N) static_cast<uint16_t*>(a.C)[row * a.ldc + col] = f32_to_bf16_bits(hv);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NJ32; ++j) {
            const int col = n0 + wn * WTN + j * 32 + (l & 31);
            if (col < a.N)
              static_cast<uint16_t*>(a.C)[row * a.ldc + col] = f32_to_bf16_bits(acc[i][j][r]);
          }
        }
      }
    }
  };
  static_assert(NI32 == 4, "row-block variants assume 4 blocks of 32 rows per wave");
  if (ni_valid > 2) body(std::integral_constant<int, 4>{});
  else if (ni_valid > 1) body(std::integral_constant<int, 2>{});
  else if (ni_valid > 0) body(std::integral_constant<int, 1>{});
  else body(std::integral_constant<int, 0>{});
}

// m-tile prefix over groups for two tile heights, one workgroup (G <= 512).
__global__ __launch_bounds__(512) void build_tiles(const int32_t* __restrict__ offsets, int E,
                                                   int Ns, int T, int TK, int bm1, int bm2,
                                                   int32_t* __restrict__ t1,
                                                   int32_t* __restrict__ t2) {
  __shared__ int s1[512], s2[512];
  const int g = threadIdx.x, G = E + Ns;
  int c1 = 0, c2 = 0;
  if (g < G) {
    int r0, r1;
    group_rows(offsets, g, E, T, TK, r0, r1);
    c1 = ceil_div(r1 - r0, bm1);
    c2 = ceil_div(r1 - r0, bm2);
  }
  s1[g] = c1;
  s2[g] = c2;
  __syncthreads();
  for (int d = 1; d < 512; d <<= 1) {
    int a1 = g >= d ? s1[g - d] : 0, a2 = g >= d ? s2[g - d] : 0;
    __syncthreads();
    s1[g] += a1;
    s2[g] += a2;
    __syncthreads();
  }
  if (g < G) {
    t1[g] = s1[g] - c1;
    t2[g] = s2[g] - c2;
  }
  if (g == G - 1) {
    t1[G] = s1[g];
    t2[G] = s2[g];
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
constexpr int kBM = 128, kBN = 128, kWM = 2, kWN = 2;      // router logits
constexpr int kEBM = 256, kEBN = 256, kEWM = 2, kEWN = 2;  // expert GEMMs

static int m_tiles_upper(const moe_config& c, int bm) {
  const long long TK = 1LL * c.num_tokens * c.top_k;
  long long routed = (TK + 1LL * c.num_experts * (bm - 1)) / bm;
  routed = routed < TK ? routed : TK;
  return int(routed + 1LL * c.num_shared * ceil_div(c.num_tokens, bm));
}

hipError_t launch_gemm_router_bf16(const moe_config& c, const uint16_t* x, const uint16_t* w,
                                   float* z, hipStream_t s) {
  GemmArgs a{};
  a.A = x;
  a.B0 = w;
  a.b_stride = 0;
  a.C = z;
  a.ldc = c.num_experts;
  a.N = c.num_experts;
  a.K = c.hidden;
  a.E = 0;
  a.T = c.num_tokens;
  a.TK = 0;
  a.G = 1;
  a.n_tiles = ceil_div(c.num_experts, kBN);
  a.k_chunk = router_k_chunk(c);
  a.c_split_stride = 1LL * c.num_tokens * c.num_experts;
  const int grid = ceil_div(c.num_tokens, kBM) * a.n_tiles;
  hipLaunchKernelGGL((grouped_gemm_bf16<kBM, kBN, kWM, kWN, kPlainF32>),
                     dim3(grid, router_splits(c)), dim3(kWM * kWN * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const moe_config& c, const int32_t* offsets, int bm1, int bm2,
                              int32_t* t1, int32_t* t2, hipStream_t s) {
  const int T = c.num_tokens, E = c.num_experts, Ns = c.num_shared;
  hipLaunchKernelGGL(build_tiles, dim3(1), dim3(512), 0, s, offsets, E, Ns, T, T * c.top_k, bm1,
                     bm2, t1, t2);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn(const moe_config& c, const void* x, const int32_t* offsets,
                              const int32_t* row_token, const moe_expert_weights& w,
                              void* y_rows, const Workspace& ws, hipStream_t s) {
  const int T = c.num_tokens, E = c.num_experts, Ns = c.num_shared;
  const int TK = T * c.top_k, G = E + Ns, rows = TK + T * Ns;
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
  if (c.w_dtype == MOE_E4M3)
    return launch_grouped_ffn_fp8(c, x, offsets, row_token, w, y_rows, ws, s);
  hipError_t err = launch_build_tiles(c, offsets, kEBM, kEBM, ws.tiles1, ws.tiles2, s);
  if (err != hipSuccess) return err;
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(x);
  a.row_token = row_token;
  a.offsets = offsets;
  a.tile_off = ws.tiles1;
  a.B0 = static_cast<const uint16_t*>(w.w_gate);
  a.B1 = static_cast<const uint16_t*>(w.w_up);
  a.b_stride = 1LL * I * H;
  a.C = ws.h;
  a.ldc = I;
  a.N = I;
  a.K = H;
  a.E = E;
  a.T = T;
  a.TK = TK;
  a.G = G;
  a.n_tiles = ceil_div(I, kEBN / 2);
  a.gather = 1;
  a.a_rows = T;
  hipLaunchKernelGGL((grouped_gemm_big<kEBM, kEBN, kEWM, kEWN, kGatedBf16>),
                     dim3(m_tiles_upper(c, kEBM) * a.n_tiles), dim3(kEWM * kEWN * 64), 0, s, a);
  GemmArgs d = a;
  d.A = static_cast<const uint16_t*>(ws.h);
  d.row_token = nullptr;
  d.gather = 0;
  d.a_rows = rows;
  d.tile_off = ws.tiles2;
  d.B0 = static_cast<const uint16_t*>(w.w_down);
  d.B1 = nullptr;
  d.b_stride = 1LL * H * I;
  d.C = y_rows;
  d.ldc = H;
  d.N = H;
  d.K = I;
  d.n_tiles = ceil_div(H, kEBN);
  hipLaunchKernelGGL((grouped_gemm_big<kEBM, kEBN, kEWM, kEWN, kPlainBf16>),
                     dim3(m_tiles_upper(c, kEBM) * d.n_tiles), dim3(kEWM * kEWN * 64), 0, s, d);
  return hipGetLastError();
}

}  // namespace moe
