// Block-scaled FP8 GEMM for gfx950 (CDNA4 MFMA): dense and grouped (MoE).
//
// C = A * B^T with A (M x K) quantized per 1x128 tile and B (N x K) per
// 128x128 block. For each 128-wide K group g the FP8 matrix cores produce the
// FP32 partial P_g of one v_mfma_f32_16x16x128_f8f6f4 (one MFMA spans exactly
// one K group), and the vector ALU promotes it into the FP32 accumulator with
// that group's scales:
//     acc[m, n] += (sa[m, g] * sb[n / 128, g]) * P_g[m, n]
// This is the per-group scaling along K and the promotion of MMA partials to
// FP32 described in "Six Reasons Deepseek Ai Is A Waste Of Time"
// (myomija.com), paragraphs on fine-grained quantization and on promotion,
// with the promotion interval read as one scale group (128).
//
// Tiling. A workgroup computes a BM x BN output tile with WAVES_M x WAVES_N
// waves; each wave owns a WM x WN sub-tile (WM = BM / WAVES_M, WN = BN /
// WAVES_N <= 128, so a wave's columns share one weight block and one sb).
// Per K group the workgroup stages the BM x 128 slab of A and the BN x 128
// slab of B in LDS. The copies go straight from global memory to LDS
// (buffer_load_dwordx4 ... lds: no VGPR round trip), into one of two stages.
// While group g multiplies, A's slab of group g+1 and B's slab of group g+2
// stream in: a wave reads its B fragments of group g+1 into registers during
// group g's last MFMAs, so B's slab of g+1 is already visible (copied during
// group g-1) and the one of g is no longer needed. A group then starts on one
// A fragment read instead of a burst of B-fragment reads by every wave. Medians
// over 20 interleaved rounds on one MI355X, same results bit for bit: 4096^3
// 62.2 -> 60.5 us, 8192x2048x7168 101.8 -> 98.5 us, 16384x4096x7168 400 ->
// 392 us, 8192x7168x2048 unchanged (119.8 / 120.1 us).
//
// A-scales: a row's scales of consecutive K groups are contiguous in sa
// (M x K/128, row-major), so the tile's scales travel in chunks of
// kScaleChunk groups (32 bytes of each row, read by 8 neighbouring lanes)
// into a two-slot ring, [row][kScaleChunk] with the column XOR-swizzled by
// row (see gemm_tile). Copying each
// group's BM scales separately touches one 128-byte line per row and group,
// as many line requests as the operand slabs themselves, and stalled the
// texture addresser; the chunked copy took 4096^3 from 63.1 to 60.9 us and
// 8192x2048x7168 from 105.9 to 102.2 us on one MI355X (same results bit
// for bit).
//
// LDS layout: rows of 128 bytes; the eight 16-byte chunks of row r are stored
// at chunk positions c ^ (r & 7), so the 16 rows read by one MFMA operand
// load fall in distinct banks. A direct-to-LDS load writes 64 consecutive
// 16-byte slots per wave instruction; each lane therefore fetches the global
// chunk that belongs in its slot.
//
// Operand lanes: for the 16x16x128 MFMA, lane l supplies row l % 16 of a
// 16-row block of B (first operand) and of A (second operand) with 32 bytes of
// K. Which 32 of the 128 K bytes a lane carries only has to agree between the
// operands: lane l takes chunks l/16 and 4 + l/16. With B first, the MFMA
// yields a block of C^T: lane l holds C[m = l % 16][n = 4 (l/16) + r],
// r = 0..3, i.e. four consecutive columns of one row. So a lane needs one row
// scale per block, and the epilogue stores 4 columns per lane at once.
//
// Ragged edges: the loads go through buffer descriptors sized to the tile's
// valid rows, so rows past the end of A (or B) read as zeros; their results
// are never stored.
//
// Row-scaled B (kRowB): for the weight-gradient GEMM both operands are
// quantized in 1x128 tiles along K, so B carries one scale per row and group,
// sb[n][g], and the promotion scale of each output element is
// sa[m, g] * sb[n, g]. The tile's BN row scales of a group are staged in LDS
// next to the A-scales, and each lane forms the four products of its four
// columns per MFMA (four extra multiplies per MFMA).
//
// Tile order is XCD-aware: the hardware hands workgroup ids to the 8 XCDs
// round-robin, so ids are remapped such that each XCD works on a contiguous
// run of tiles (neighbouring tiles share A rows / B columns in its L2).
#include <atomic>

#include "common.hpp"
#include "tiles.hpp"

namespace fp8q {

struct GemmArgs {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;           // 128x128 block scales, or N x G row scales (kRowB)
  void* c;
  const int32_t* m_offsets;  // grouped only
  int M;                     // rows of A / C (M_total when grouped)
  int N;
  int K;
  int G;        // experts (grouped); 1 for dense
  int n_tiles;  // number of real tiles (dense) / upper bound (grouped)
  int n_big;      // dense with a tail: workgroups of 256 x 256 tiles (columns [0, n_col_main))
  int n_col_main; // dense with a tail: the remaining columns go in 256 x 128 tiles
};

// K groups per A-scale chunk (8 groups: 32 bytes of each row's scales)
constexpr int kScaleChunk = 8;
// A wave's own LDS writes are complete, and neither the compiler nor the
// hardware moves its later LDS reads (of what other lanes wrote) ahead of them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Scale-ring column swizzle of row r (see the ring's layout in gemm_tile)
__device__ __forceinline__ int ring_swz(int r) { return (r >> 2) & 3; }

template <int BM, int BN, int WAVES_M, int WAVES_N, bool kRowB = false>
struct TileCfg {
  static constexpr int kWM = BM / WAVES_M;
  static constexpr int kWN = BN / WAVES_N;
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kSubM = kWM / 16;
  static constexpr int kSubN = kWN / 16;
  static constexpr int kLdsA = BM * 128;  // bytes per stage
  static constexpr int kLdsB = BN * 128;
  static constexpr int kStage = kLdsA + kLdsB;
  // scale ring: rows whose per-group scales are staged (A rows; with kRowB
  // also B's rows), kScaleChunk groups per slot, two slots
  static constexpr int kScaleRows = BM + (kRowB ? BN : 0);
  static constexpr int kSlot = kScaleRows * kScaleChunk * 4;
  static constexpr int kScaleCopies = kSlot / 4 / kThreads;  // scales per thread per chunk
  static constexpr int kLdsBytes = 2 * kStage + 2 * kSlot;
  static constexpr int kLoadsA = BM * 8 / kThreads;  // 16-byte chunks per thread per group
  static constexpr int kLoadsB = BN * 8 / kThreads;
  static_assert(kWN <= 128 && 128 % kWN == 0, "a wave's columns must share one weight block");
  static_assert(BM * 8 % kThreads == 0 && BN * 8 % kThreads == 0, "whole wave loads");
  static_assert(kSlot % (4 * kThreads) == 0 && BM * kScaleChunk * 4 % (4 * kThreads) == 0,
                "scale chunks: whole copies per thread, A and B rows in separate copies");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};


// One BM x BN output tile: `tile` numbers the tiles of the columns
// [col_base, col_end) (dense) or of all experts (grouped); `lds` holds at
// least TileCfg::kLdsBytes (two stages, the scale ring; the epilogue's staging).
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kBf16Out, bool kGrouped, bool kRowB>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, uint8_t* __restrict__ lds, int tile,
                                          int col_base, int col_end) {
  using Cfg = TileCfg<BM, BN, WAVES_M, WAVES_N, kRowB>;
  static_assert(!(kGrouped && kRowB), "row-scaled B is dense only");
  constexpr int WM = Cfg::kWM, WN = Cfg::kWN;
  constexpr int SUBM = Cfg::kSubM, SUBN = Cfg::kSubN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int G = p.K / kGroup;
  const int n_tiles_n = (col_end - col_base + BN - 1) / BN;

  // ---- tile -> (rows [m0, m_end), columns n0, expert) ----
  int m0, m_end, tile_n;
  const uint8_t* bmat = p.b;
  const float* sbmat = p.sb;
  if constexpr (kGrouped) {
    // tiles are numbered expert by expert (ceil(rows_e / BM) x n_tiles_n each),
    // banded within an expert. The tile's expert: one expert per lane, 64 per
    // round, an inclusive prefix of their tile counts across the lanes, and
    // the first lane whose prefix passes the tile; its values are read back
    // with readlane, so they stay scalar (lane shuffles would make them vector
    // values, and every buffer descriptor built from them a loop). A loop over
    // the experts one by one cost 2.8% with 70 experts (1969.5 against
    // 2026.9 us, same results bit for bit; unchanged with 32).
    int e = -1, before = 0, lo = 0, hi = 0, te = 0;
    for (int e0 = 0; e0 < p.G; e0 += 64) {
      const int ee = e0 + lane;
      int l_lo = 0, l_hi = 0, l_te = 0;
      if (ee < p.G) {
        l_lo = min(max(p.m_offsets[ee], 0), p.M);
        l_hi = min(max(p.m_offsets[ee + 1], l_lo), p.M);
        l_te = (l_hi - l_lo + BM - 1) / BM;
      }
      const int cnt = l_te * n_tiles_n;
      int incl = cnt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
      }
      const uint64_t hit = __ballot(ee < p.G && tile < before + incl);
      if (hit) {
        const int L = __builtin_ctzll(hit);
        e = e0 + L;
        lo = __builtin_amdgcn_readlane(l_lo, L);
        hi = __builtin_amdgcn_readlane(l_hi, L);
        te = __builtin_amdgcn_readlane(l_te, L);
        before += __builtin_amdgcn_readlane(incl - cnt, L);
        break;
      }
      before += __builtin_amdgcn_readlane(incl, 63);
    }
    if (e < 0) return;  // beyond the last real tile (grid is an upper bound)
    int tm;
    band_tile<kBandGrouped>(tile - before, te, n_tiles_n, tm, tile_n);
    m0 = lo + tm * BM;
    m_end = min(m0 + BM, hi);
    bmat += (int64_t)e * p.N * p.K;
    sbmat += (int64_t)e * (p.N / kGroup) * G;
  } else {
    int tm;
    band_tile(tile, (p.M + BM - 1) / BM, n_tiles_n, tm, tile_n);
    m0 = tm * BM;
    m_end = min(m0 + BM, p.M);
  }
  const int n0 = col_base + tile_n * BN;
  const int n_last = p.N - 1;

  // ---- global -> LDS copies through buffer descriptors ----
  // One descriptor per operand covers exactly the tile's valid rows, so rows
  // past the end of A (or B) read as zeros. Their outputs are never stored;
  // every output row depends only on its own A row. Slot s = i * kThreads +
  // tid of a stage holds row s / 8, stored chunk s % 8, i.e. the global chunk
  // (s % 8) ^ (row % 8); the per-group advance (g * 128 bytes) is the
  // instruction's scalar offset.
  const int rows_a = m_end - m0;
  const int rows_b = min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(p.a + (int64_t)m0 * p.K, (uint32_t)rows_a * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(bmat + (int64_t)n0 * p.K, (uint32_t)rows_b * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t rsrc_sa = make_rsrc(p.sa + (int64_t)m0 * G, (uint32_t)rows_a * (uint32_t)G * 4);
  __amdgpu_buffer_rsrc_t rsrc_sbr = rsrc_sa;  // kRowB: B's row scales over the tile's valid columns
  if constexpr (kRowB)
    rsrc_sbr = make_rsrc(p.sb + (int64_t)n0 * G, (uint32_t)rows_b * (uint32_t)G * 4);
  // Scale ring slot: row r's kScaleChunk scales in 32 bytes, scale c at
  // position c ^ ring_swz(r). The readers of one scale column are the 16 rows
  // of a 16-row block (A) or rows 4 apart (kRowB's B rows); with the XOR the
  // 16 A rows fall in 16 distinct banks instead of four rows per bank.
  // Copy q of thread tid fills slot position q * kThreads + tid: row
  // q * kThreads / 8 + tid / 8, position tid % 8, i.e. the scale
  // (tid % 8) ^ ring_swz(row). The row part stays in the per-lane offset,
  // where the buffer range check covers it: rows past the valid ones read as
  // zeros (groups past G, never used, read the next row's first scales).
  static_assert(Cfg::kThreads % 128 == 0, "ring_swz(row) is the same for every copy of a thread");
  const uint32_t sc_row_off =
      (uint32_t)(tid >> 3) * (uint32_t)G * 4 + (uint32_t)(((tid & 7) ^ ring_swz(tid >> 3)) * 4);
  static_assert(!kRowB || BN == BM, "B rows fill whole copies");
  uint8_t* const ring = lds + 2 * Cfg::kStage;
  // chunk `chunk` of the tile's scales into its ring slot
  auto issue_scales = [&](int chunk, uint8_t* __restrict__ slot) {
    const uint32_t off = sc_row_off + (uint32_t)chunk * (kScaleChunk * 4);
#pragma unroll
    for (int q = 0; q < Cfg::kScaleCopies; ++q) {
      // copies of A rows first (q * kThreads < 8 BM), then B rows (kRowB)
      const bool a_rows = q * Cfg::kThreads < 8 * BM;
      const uint32_t row_base = a_rows ? (uint32_t)(q * Cfg::kThreads / 8) : (uint32_t)(q * Cfg::kThreads / 8 - BM);
      load_lds(a_rows ? rsrc_sa : rsrc_sbr, slot + (q * Cfg::kThreads + wave * 64) * 4, 4,
               off + row_base * (uint32_t)G * 4, 0);
    }
  };
  // Slot q * kThreads + tid has row q * (kThreads / 8) + tid / 8 and stored
  // chunk tid % 8, so copy q's per-lane offset is offa + q * row_step. The row
  // part must stay in the per-lane offset: the buffer range check covers the
  // per-lane offset but not the scalar one (which only carries the group's
  // advance inside a row).
  static_assert(Cfg::kThreads % 64 == 0, "row step keeps row % 8");
  const int row0 = tid >> 3, lc0 = (tid & 7) ^ (row0 & 7);
  const uint32_t offa = (uint32_t)row0 * (uint32_t)p.K + lc0 * 16;
  const uint32_t offb = offa;
  const uint32_t row_step = (uint32_t)(Cfg::kThreads / 8) * (uint32_t)p.K;

  // Copy number q (0 .. kCopies-1) of this thread's share of the slabs: the
  // first kLoadsA copies bring A's slab of group ga into stage sta, the rest
  // B's slab of group gb into stage stb.
  constexpr int kCopies = Cfg::kLoadsA + Cfg::kLoadsB;
  auto issue_copy = [&](int q, int ga, uint8_t* __restrict__ sta, int gb, uint8_t* __restrict__ stb) {
    if (q < Cfg::kLoadsA) {
      load_lds(rsrc_a, sta + (q * Cfg::kThreads + wave * 64) * 16, 16, offa + q * row_step,
               ga * kGroup);
    } else {
      const int i = q - Cfg::kLoadsA;
      load_lds(rsrc_b, stb + Cfg::kLdsA + (i * Cfg::kThreads + wave * 64) * 16, 16,
               offb + i * row_step, gb * kGroup);
    }
  };
  auto issue_loads = [&](int ga, uint8_t* __restrict__ sta, int gb, uint8_t* __restrict__ stb) {
#pragma unroll
    for (int q = 0; q < kCopies; ++q) issue_copy(q, ga, sta, gb, stb);
  };

  v4f acc[SUBM][SUBN];
#pragma unroll
  for (int i = 0; i < SUBM; ++i)
#pragma unroll
    for (int j = 0; j < SUBN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15;  // operand row within a 16-row block
  const int lk = lane >> 4;  // which 16-byte chunk pair of the group
  const int nb = min(n0 + wn * WN, n_last) / kGroup;
  const float* gsb = sbmat + (int64_t)nb * G;

  // Operand fragment of the 16-row block starting at `blk` (a row index that
  // is a multiple of 16, so row % 8 == lr % 8): the lane's two chunks sit at
  // fixed per-lane offsets from the block start.
  const int lane_lo = lr * 128 + ((lk ^ (lr & 7)) << 4);
  const int lane_hi = lr * 128 + (((4 + lk) ^ (lr & 7)) << 4);
  auto load_frag = [&](const uint8_t* blk) {
    const uint4 lo = *(const uint4*)(blk + lane_lo);
    const uint4 hi = *(const uint4*)(blk + lane_hi);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  // One pipeline step: multiply the K group whose A slab is at sA (sbv: its
  // weight scale) with the B fragments held in bf, read the next group's B
  // fragments from sBn into bf, and copy A's slab of group ga into nxt and
  // B's slab of group gb into cur_w. The restrict-qualified pointers tell the
  // compiler (and its wait-count pass) that the LDS reads never alias the
  // in-flight copies, so those copies are not waited on until the barrier.
  //
  // The step's instruction order is fixed in the source: scheduling barriers
  // around each MFMA keep the compiler from moving anything across it. Left
  // free, the scheduler placed some promotion FMAs ahead of the next MFMA, on
  // the result of the MFMA just issued: the wave then waited out that MFMA's
  // whole latency before it could issue the next one (14 of the 128 FMAs of
  // a step, plus 109 cycles of hazard s_nops). The FMAs promoting an MFMA are
  // issued after the MFMA kPromoteLag places later, so each promotion reads a
  // result that is already complete and needs no wait states (12 s_nop
  // cycles per step). Measured on MI355X in one process, same results bit
  // for bit: 4096^3 61.5 -> 58.4 us, 8192x2048x7168 101.0 -> 95.9 us,
  // 8192x7168x2048 117.2 -> 114.8 us. A lag of 3 and A-fragment reads two
  // blocks ahead measured the same or slower. With 128x128 weight blocks the
  // last kPromoteLag results of a step are promoted during the next step's
  // first MFMAs (their scales and results carried over), so a wave reaches
  // the group's barrier without waiting for its last MFMA: 0.5-1.3% faster
  // on the same four shapes.
  //
  // The copies are spread over the MFMAs (one every kCopyEvery MFMAs): a wave
  // issues in order, and a burst of direct-to-LDS copies would hold back its
  // MFMAs while the memory pipeline accepts them. They start before MFMA
  // kCopyOff. The dense GEMM does best with one copy every 2 MFMAs from MFMA 3
  // (offsets 1, 2, 5 and spacings 1, 3 measured the same or up to 2% slower).
  // The grouped GEMM, whose weights come from HBM rather than the Infinity
  // Cache, wants its copies as early as possible: one per MFMA from MFMA 0
  // (32-expert MoE: 1860 us, against 1878, 1896 and 1921 us from MFMA 1, 2
  // and 3). The dense tail's half-width tiles (16 MFMAs per step) do best
  // with one copy per MFMA from MFMA 1: 8192x7168x2048 111.7 -> 109.8 us,
  // 4000x4352x2048 47.5 -> 46.7 us (from MFMA 0, every 1 or 2, and from
  // MFMA 2 every 2: 110.3-111.5 and 45.9-47.3 us).
  constexpr bool kHalfWidth = !kGrouped && BN == 128;
  constexpr int kCopyOff = kGrouped ? 0 : (kHalfWidth ? 1 : 3);
  constexpr int kCopyEvery = kGrouped || kHalfWidth ? 1 : 2;
  constexpr int kPromoteLag = 2;
  static_assert(kCopyOff + (kCopies - 1) * kCopyEvery < SUBM * SUBN, "the copies fit in a step");
  // acc += part * scale: one scale for the lane's four columns (128x128 B
  // blocks: sc1 = sa * sb), or one per column (kRowB: sa * sb_row, formed
  // here so that no per-column products stay live across MFMAs)
  auto promote = [](v4f& c, const v4f& part, float sc1, float sa1, const v4f& sbr) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c[r] = __builtin_fmaf(part[r], kRowB ? sbr[r] * sa1 : sc1, c[r]);
  };
  v8i bf[SUBN];  // B fragments of the group being computed
  // kCarry: the last kPromoteLag MFMA results of a step, and the scale
  // products of its row blocks, stay live into the next step, which promotes
  // them after its first MFMAs (and the loop's end after the last step). The
  // row-scaled path (per-column B scales) promotes them within the step.
  constexpr bool kCarry = !kRowB;
  float scb_c[SUBM];
  v4f pend_c[kPromoteLag];
#pragma unroll
  for (int i = 0; i < SUBM; ++i) scb_c[i] = 0.0f;  // the first step promotes zeros
#pragma unroll
  for (int i = 0; i < kPromoteLag; ++i) pend_c[i] = v4f{0.f, 0.f, 0.f, 0.f};
  // row block and column block of the step's MFMA number t
  auto mfma_i = [](int t) {
    constexpr int kTail0 = (SUBM - 2) * SUBN;
    return t < kTail0 ? t / SUBN : SUBM - 2 + (t - kTail0) % 2;
  };
  auto mfma_j = [](int t) {
    constexpr int kTail0 = (SUBM - 2) * SUBN;
    return t < kTail0 ? t % SUBN : (t - kTail0) / 2;
  };
  // sslot, gc: the ring slot holding this group's scales and the group's
  // column in it; chunk >= 0: copy that scale chunk into `nslot` during this step.
  auto step = [&](const uint8_t* __restrict__ sA, const uint8_t* __restrict__ sBn,
                  uint8_t* __restrict__ nxt, int ga, uint8_t* __restrict__ cur_w, int gb,
                  float sbv, const float* __restrict__ sslot, int gc, int chunk,
                  uint8_t* __restrict__ nslot) {
    // the lane's A rows are wm * WM + 16 i + lr: ring_swz(row) = ring_swz(lr)
    const float* sSa = sslot + (wm * WM + lr) * kScaleChunk + (gc ^ ring_swz(lr));
    // kRowB: the row scales of the lane's four columns in each 16-column block
    v4f sbq[kRowB ? SUBN : 1];
    if constexpr (kRowB) {
      // rows BM + wn * WN + 16 j + 4 lk + r, r < 4: ring_swz(row) = ring_swz(4 lk)
      const float* sSb = sslot + (BM + wn * WN + 4 * lk) * kScaleChunk + (gc ^ ring_swz(4 * lk));
#pragma unroll
      for (int j = 0; j < SUBN; ++j)
        sbq[j] = v4f{sSb[(j * 16) * kScaleChunk], sSb[(j * 16 + 1) * kScaleChunk],
                     sSb[(j * 16 + 2) * kScaleChunk], sSb[(j * 16 + 3) * kScaleChunk]};
    }
    // MFMA order: 16-row blocks 0 .. SUBM-3 row by row, then the last two
    // blocks column by column, so that B fragment j is free (and the next
    // group's fragment j is read into it) from the 2j+2-th MFMA of that tail
    // on. The A fragment and A-scale of block b are read during block b-1
    // (block SUBM-1's during block SUBM-3).
    static_assert(SUBM >= 3 && SUBN >= 3, "three 16-row blocks and 16-column blocks");
    constexpr int kTail0 = (SUBM - 2) * SUBN;
    v8i af[SUBM];
    float sav[SUBM];
    float scb_l[kCarry ? 1 : SUBM];
    float* const scb = kCarry ? scb_c : scb_l;
    af[0] = load_frag(sA + wm * WM * 128);
    sav[0] = sSa[0];
    // MFMA results not yet promoted: that of MFMA t sits in slot t % kPromoteLag
    v4f pend_l[kCarry ? 1 : kPromoteLag];
    v4f* const pend = kCarry ? pend_c : pend_l;
    auto promote_pending = [&](int tp) {
      const int pi = mfma_i(tp), pj = mfma_j(tp);
      promote(acc[pi][pj], pend[tp % kPromoteLag], scb[pi], sav[pi], sbq[kRowB ? pj : 0]);
    };
#pragma unroll
    for (int t = 0; t < SUBM * SUBN; ++t) {
      const int i = mfma_i(t);
      const int j = mfma_j(t);
      const bool first_of_block = t < kTail0 ? j == 0 : t - kTail0 < 2;
      if (t >= kCopyOff && (t - kCopyOff) % kCopyEvery == 0 && (t - kCopyOff) / kCopyEvery < kCopies)
        issue_copy((t - kCopyOff) / kCopyEvery, ga, nxt, gb, cur_w);
      if (t == 1 && chunk >= 0) issue_scales(chunk, nslot);
      if (t < kTail0 && j == 0 && i + 1 <= SUBM - 2) {
        af[i + 1] = load_frag(sA + (wm * WM + (i + 1) * 16) * 128);
        sav[i + 1] = sSa[(i + 1) * 16 * kScaleChunk];
      }
      if (t == kTail0 - SUBN + 2) {
        af[SUBM - 1] = load_frag(sA + (wm * WM + (SUBM - 1) * 16) * 128);
        sav[SUBM - 1] = sSa[(SUBM - 1) * 16 * kScaleChunk];
      }
      if (first_of_block) scb[i] = sav[i] * sbv;
      const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          bf[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // block SUBM-1 is B fragment j's last use: read the next group's
      if (i == SUBM - 1) bf[j] = load_frag(sBn + (wn * WN + j * 16) * 128);
      if (t >= kPromoteLag) {
        promote_pending(t - kPromoteLag);
      } else if constexpr (kCarry) {
        // the previous step's MFMA SUBM * SUBN - kPromoteLag + t (zeros in the first step)
        promote_pending(SUBM * SUBN - kPromoteLag + t);
      }
      pend[t % kPromoteLag] = part;
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!kCarry) {
#pragma unroll
      for (int t = SUBM * SUBN - kPromoteLag; t < SUBM * SUBN; ++t) promote_pending(t);
    }
  };

  // A wave whose 16-row blocks all lie past the tile's valid rows (the
  // 128-row remainder of an expert, a ragged last row tile) only copies its
  // share of each group and keeps the barriers; its MFMAs would multiply the
  // zero rows. The other wave of its SIMD then has the matrix core alone.
  const bool idle = wm * WM >= rows_a;

  // ---- main loop: group g computes from A's slab in stage g % 2 and B fragments
  // held in registers, while A's slab of g+1 streams into the other stage and
  // B's slab of g+2 into stage g % 2 (B's slab of g was read a group ago) ----
  // Scale chunk c (groups kScaleChunk c ..) lives in ring slot c % 2. Chunk
  // c + 1 is copied during the first step of chunk c, into the slot chunk
  // c - 1 used: every wave finished chunk c - 1's last group before the
  // barrier that ends it.
  float sbv = 0.0f;
  if (G > 0) {
    if constexpr (!kRowB) sbv = gsb[0];
    issue_loads(0, lds, 0, lds);
#pragma unroll
    for (int q = Cfg::kLoadsA; q < kCopies; ++q) issue_copy(q, 0, lds, min(1, G - 1), lds + Cfg::kStage);
    issue_scales(0, ring);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (!idle) {
#pragma unroll
    for (int j = 0; j < SUBN; ++j) bf[j] = load_frag(lds + Cfg::kLdsA + (wn * WN + j * 16) * 128);
  }
  // the first step copies B's slab of group 2 over the one just read
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    uint8_t* cur = lds + (g & 1) * Cfg::kStage;
    uint8_t* nxt = lds + ((g + 1) & 1) * Cfg::kStage;
    const int c = g / kScaleChunk;
    const int next_chunk = (g % kScaleChunk == 0 && (c + 1) * kScaleChunk < G) ? c + 1 : -1;
    uint8_t* nslot = ring + ((c + 1) & 1) * Cfg::kSlot;
    const float* sslot = (const float*)(ring + (c & 1) * Cfg::kSlot);
    const float sbv_next = (!kRowB && g + 1 < G) ? gsb[g + 1] : 0.0f;
    // past the last group the copies repeat group G-1 into slabs never read
    // again (and the last step's B-fragment reads are unused): no branch in the step
    if (idle) {
      issue_loads(min(g + 1, G - 1), nxt, min(g + 2, G - 1), cur);
      if (next_chunk >= 0) issue_scales(next_chunk, nslot);
    } else {
      step(cur, nxt + Cfg::kLdsA, nxt, min(g + 1, G - 1), cur, min(g + 2, G - 1), sbv, sslot,
           g % kScaleChunk, next_chunk, nslot);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this thread's copies have landed
    __syncthreads();                     // ... and everyone's; `cur` is free again
    sbv = sbv_next;
  }
  if constexpr (kCarry) {
    if (!idle) {
#pragma unroll
      for (int t = SUBM * SUBN - kPromoteLag; t < SUBM * SUBN; ++t)
        promote(acc[mfma_i(t)][mfma_j(t)], pend_c[t % kPromoteLag], scb_c[mfma_i(t)], 0.0f,
                v4f{0.f, 0.f, 0.f, 0.f});
    }
  }

  // ---- epilogue ----
  if constexpr (kBf16Out) {
    // The MFMA layout gives a lane 4 columns (8 bytes) of one row, so direct
    // stores would write every 128-byte line in four 32-byte pieces. Instead
    // each wave stages its WM x WN tile in its own part of the (now idle) LDS
    // and stores whole 128-byte row segments, 16 bytes per lane. LDS rows are
    // 128 bytes with the 16-byte chunk index XOR row % 8, so the staging
    // writes of 16 rows hit distinct banks pairwise and the reads are
    // conflict-free. The loop above ends with a barrier, so no wave still
    // reads the stages; each wave then reads back only what it wrote itself
    // (a wave's LDS accesses are processed in order), so no barrier is needed
    // between the staging writes and the reads, and a wave that finishes its
    // MFMAs first starts storing first.
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    static_assert(WN * 2 == 128, "one 128-byte row segment per wave row");
    static_assert(WAVES_M * WAVES_N * WM * 128 <= Cfg::kLdsBytes, "staging fits in the stages");
    uint8_t* tile = lds + wave * (WM * 128);
#pragma unroll
    for (int i = 0; i < SUBM; ++i) {
      const int m = i * 16 + lr;
#pragma unroll
      for (int j = 0; j < SUBN; ++j) {
        const int byte = j * 32 + lk * 8;  // column (j * 16 + 4 * lk) * 2 bytes
        const bf16x4 v = {(__bf16)acc[i][j][0], (__bf16)acc[i][j][1], (__bf16)acc[i][j][2],
                          (__bf16)acc[i][j][3]};
        *(bf16x4*)(tile + m * 128 + ((((byte >> 4) ^ (m & 7))) << 4) + (byte & 15)) = v;
      }
    }
    wave_lds_sync();
    const int nw = n0 + wn * WN;  // N % 128 == 0: the wave's 64 columns are all in or all out
    if (nw < p.N) {
      const int c = lane & 7;
#pragma unroll
      for (int k = 0; k < WM / 8; ++k) {
        const int m = k * 8 + (lane >> 3);
        const int gm = m0 + wm * WM + m;
        const uint4 v = *(const uint4*)(tile + m * 128 + ((c ^ (m & 7)) << 4));
        if (gm < m_end) *(uint4*)((__bf16*)p.c + (int64_t)gm * p.N + nw + c * 8) = v;
      }
    }
  } else {
    // FP32: the same wave-local staging in two passes of WM / 2 rows (a row
    // is 256 bytes, 16 chunks of 16 bytes at chunk index XOR row % 16); the
    // second pass's writes follow the first pass's reads in the wave's order
    static_assert(WN * 4 == 256 && SUBM % 2 == 0, "two passes of 256-byte rows");
    static_assert(WAVES_M * WAVES_N * (WM / 2) * 256 <= Cfg::kLdsBytes, "staging fits in the stages");
    uint8_t* tile = lds + wave * ((WM / 2) * 256);
    const int nw = n0 + wn * WN;
    const int c = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < SUBM / 2; ++i) {
        const int m = i * 16 + lr;
#pragma unroll
        for (int j = 0; j < SUBN; ++j)
          *(v4f*)(tile + m * 256 + (((j * 4 + lk) ^ (m & 15)) << 4)) = acc[h * (SUBM / 2) + i][j];
      }
      wave_lds_sync();
      if (nw < p.N) {
#pragma unroll
        for (int k = 0; k < WM / 8; ++k) {
          const int m = k * 4 + (lane >> 4);
          const int gm = m0 + wm * WM + h * (WM / 2) + m;
          const v4f v = *(const v4f*)(tile + m * 256 + ((c ^ (m & 15)) << 4));
          if (gm < m_end) *(v4f*)((float*)p.c + (int64_t)gm * p.N + nw + c * 4) = v;
        }
      }
    }
  }
}


// The workgroup's tile. With a tail (dense, kTail), workgroups n_big.. take
// 256 x 128 tiles of the columns [n_col_main, N): a last, partly filled wave
// of 256 x 256 tiles becomes a full wave of tiles half as long, all in one
// launch. Each part's tile order is XCD-aware on its own.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kBf16Out, bool kGrouped, bool kRowB, bool kTail>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_blockscaled_kernel(GemmArgs p) {
  using Cfg = TileCfg<BM, BN, WAVES_M, WAVES_N, kRowB>;
  using TailCfg = TileCfg<BM, kTail ? BN / 2 : BN, kTail ? 2 * WAVES_M : WAVES_M,
                          kTail ? WAVES_N / 2 : WAVES_N, kRowB>;
  static_assert(!kTail || (!kGrouped && TailCfg::kThreads == Cfg::kThreads), "tail: dense, same workgroup");
  constexpr int kLds = (kTail && TailCfg::kLdsBytes > Cfg::kLdsBytes) ? TailCfg::kLdsBytes : Cfg::kLdsBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  if constexpr (kTail) {
    // Workgroups in three runs: h1 of the half-width tiles, all full tiles,
    // the other half-width tiles. The CUs that start on a half-width tile run
    // half a tile ahead of the others from then on, so each wave of tiles ends
    // (and writes its output) in two groups half a tile apart instead of all
    // at once. Runs start at multiples of 8 ids where the counts allow, which
    // keeps each run's tile order XCD-aware.
    const int id = (int)blockIdx.x;
    const int n_half = (int)gridDim.x - p.n_big;
    const int h1 = (n_half / 2) & ~(kXcds - 1);
    if (id < h1) {
      gemm_tile<BM, BN / 2, 2 * WAVES_M, WAVES_N / 2, kBf16Out, kGrouped, kRowB>(
          p, lds, xcd_tile(id, h1), p.n_col_main, p.N);
    } else if (id < h1 + p.n_big) {
      gemm_tile<BM, BN, WAVES_M, WAVES_N, kBf16Out, kGrouped, kRowB>(
          p, lds, xcd_tile(id - h1, p.n_big), 0, p.n_col_main);
    } else {
      gemm_tile<BM, BN / 2, 2 * WAVES_M, WAVES_N / 2, kBf16Out, kGrouped, kRowB>(
          p, lds, h1 + xcd_tile(id - h1 - p.n_big, n_half - h1), p.n_col_main, p.N);
    }
  } else {
    gemm_tile<BM, BN, WAVES_M, WAVES_N, kBf16Out, kGrouped, kRowB>(
        p, lds, xcd_tile(blockIdx.x, gridDim.x), 0, p.N);
  }
}

// ---------------------------------------------------------------------------
// Small-M GEMM (HBM-bound shapes such as 64 x 7168 x 7168). A workgroup owns a
// 64 x 32 block of C; its 8 waves split the K groups between them, each wave
// streaming its B and A fragments straight from global memory into registers,
// one group ahead, and promoting its own partial sums. The 8 partial blocks
// are then summed through LDS (a fixed order, so results are deterministic)
// and stored. B is read exactly once; A (small) is re-read per column block
// from L2.
// ---------------------------------------------------------------------------
constexpr int kSkM = 64;     // rows per workgroup
constexpr int kSkN = 32;     // columns per workgroup
constexpr int kSkWaves = 8;  // K split inside the workgroup

struct SkinnyFrags {
  v8i b[kSkN / 16];
  v8i a[kSkM / 16];
  float sa[kSkM / 16];
  float sb;
};

// kRowB: the row scales of the lane's four columns in each 16-column block
template <bool kRowB>
struct SkinnyRowScales {
  v4f sb[kSkN / 16];
};
template <>
struct SkinnyRowScales<false> {};

template <bool kBf16Out, bool kRowB>
__global__ __launch_bounds__(64 * kSkWaves) void gemm_skinny_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) float part[kSkWaves][(kSkM / 16) * (kSkN / 16)][64][4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lk = lane >> 4;
  const int G = p.K / kGroup;
  const int n_blocks = p.N / kSkN;
  const int nb_idx = blockIdx.x % n_blocks;
  const int m0 = (blockIdx.x / n_blocks) * kSkM;
  const int n0 = nb_idx * kSkN;

  // this wave's K groups: a contiguous range
  const int g_begin = (int)((int64_t)G * wave / kSkWaves);
  const int g_end = (int)((int64_t)G * (wave + 1) / kSkWaves);

  // Operands through buffer descriptors over the workgroup's rows, with
  // 32-bit per-lane row offsets and the group's advance inside a row as the
  // scalar offset (the range check covers the per-lane part, so A rows past
  // M read as zeros; their outputs are never stored). All kSkN B rows exist
  // (N % 128 == 0).
  const int rows_a = min(kSkM, p.M - m0);
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(p.a + (int64_t)m0 * p.K, (uint32_t)rows_a * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t rsrc_sa = make_rsrc(p.sa + (int64_t)m0 * G, (uint32_t)rows_a * (uint32_t)G * 4);
  const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(p.b + (int64_t)n0 * p.K, (uint32_t)kSkN * (uint32_t)p.K);
  // block scales: the G scales of weight block n0 / 128; row scales (kRowB):
  // rows n0 .. n0 + kSkN - 1, G each
  const __amdgpu_buffer_rsrc_t rsrc_sb =
      kRowB ? make_rsrc(p.sb + (int64_t)n0 * G, (uint32_t)kSkN * (uint32_t)G * 4)
            : make_rsrc(p.sb + (int64_t)(n0 / kGroup) * G, (uint32_t)G * 4);
  uint32_t a_off[kSkM / 16], sa_off[kSkM / 16], b_off[kSkN / 16];
#pragma unroll
  for (int ib = 0; ib < kSkM / 16; ++ib) {
    a_off[ib] = (uint32_t)(ib * 16 + lr) * (uint32_t)p.K + lk * 16;
    sa_off[ib] = (uint32_t)(ib * 16 + lr) * (uint32_t)G * 4;
  }
#pragma unroll
  for (int jb = 0; jb < kSkN / 16; ++jb) b_off[jb] = (uint32_t)(jb * 16 + lr) * (uint32_t)p.K + lk * 16;
  // kRowB: the lane's columns are n0 + 16 jb + 4 lk + r, r = 0..3
  const uint32_t sbr_off = (uint32_t)(4 * lk) * (uint32_t)G * 4;
  const uint32_t sb_row_step = (uint32_t)G * 4;

  auto frag = [](u32x4 lo, u32x4 hi) {
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto load = [&](int g, SkinnyFrags& f, SkinnyRowScales<kRowB>& fr) {
    const int ko = g * kGroup;
#pragma unroll
    for (int jb = 0; jb < kSkN / 16; ++jb)
      f.b[jb] = frag(__builtin_amdgcn_raw_buffer_load_b128(rsrc_b, b_off[jb], ko, 0),
                     __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, b_off[jb], ko + 64, 0));
#pragma unroll
    for (int ib = 0; ib < kSkM / 16; ++ib) {
      f.a[ib] = frag(__builtin_amdgcn_raw_buffer_load_b128(rsrc_a, a_off[ib], ko, 0),
                     __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, a_off[ib], ko + 64, 0));
      f.sa[ib] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_sa, sa_off[ib], g * 4, 0));
    }
    if constexpr (kRowB) {
#pragma unroll
      for (int jb = 0; jb < kSkN / 16; ++jb) {
        v4f v;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rsrc_sb, sbr_off, (jb * 16 + r) * sb_row_step + g * 4, 0));
        fr.sb[jb] = v;
      }
    } else {
      f.sb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_sb, 0, g * 4, 0));
    }
  };

  v4f acc[kSkM / 16][kSkN / 16];
#pragma unroll
  for (int ib = 0; ib < kSkM / 16; ++ib)
#pragma unroll
    for (int jb = 0; jb < kSkN / 16; ++jb) acc[ib][jb] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const SkinnyFrags& f, const SkinnyRowScales<kRowB>& fr) {
#pragma unroll
    for (int ib = 0; ib < kSkM / 16; ++ib) {
#pragma unroll
      for (int jb = 0; jb < kSkN / 16; ++jb) {
        v4f sc;
        if constexpr (kRowB) {
          sc = fr.sb[jb] * f.sa[ib];
        } else {
          const float s1 = f.sa[ib] * f.sb;
          sc = v4f{s1, s1, s1, s1};
        }
        const v4f pp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            f.b[jb], f.a[ib], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        acc[ib][jb][0] = __builtin_fmaf(pp[0], sc[0], acc[ib][jb][0]);
        acc[ib][jb][1] = __builtin_fmaf(pp[1], sc[1], acc[ib][jb][1]);
        acc[ib][jb][2] = __builtin_fmaf(pp[2], sc[2], acc[ib][jb][2]);
        acc[ib][jb][3] = __builtin_fmaf(pp[3], sc[3], acc[ib][jb][3]);
      }
    }
  };

  // two register stages: group g+1 is in flight while g is multiplied
  SkinnyFrags f0, f1;
  SkinnyRowScales<kRowB> r0, r1;
  int g = g_begin;
  if (g < g_end) load(g, f0, r0);
  for (; g + 1 < g_end; g += 2) {
    load(g + 1, f1, r1);
    compute(f0, r0);
    if (g + 2 < g_end) load(g + 2, f0, r0);
    compute(f1, r1);
  }
  if (g < g_end) compute(f0, r0);

  // ---- reduce the waves' partial blocks in LDS, in wave order ----
#pragma unroll
  for (int ib = 0; ib < kSkM / 16; ++ib)
#pragma unroll
    for (int jb = 0; jb < kSkN / 16; ++jb)
      *(v4f*)part[wave][ib * (kSkN / 16) + jb][lane] = acc[ib][jb];
  __syncthreads();
  constexpr int kBlocks = (kSkM / 16) * (kSkN / 16);
  static_assert(kBlocks * 64 == 64 * kSkWaves, "one output quad per thread");
  const int blk = tid >> 6;  // block of this thread's quad
  v4f sum = *(const v4f*)part[0][blk][lane];
#pragma unroll
  for (int w = 1; w < kSkWaves; ++w) sum += *(const v4f*)part[w][blk][lane];
  const int ib = blk / (kSkN / 16), jb = blk % (kSkN / 16);
  const int gm = m0 + ib * 16 + lr;
  const int gn = n0 + jb * 16 + 4 * lk;
  if (gm < p.M) {
    const int64_t off = (int64_t)gm * p.N + gn;
    if constexpr (kBf16Out) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 v = {(__bf16)sum[0], (__bf16)sum[1], (__bf16)sum[2], (__bf16)sum[3]};
      *(bf16x4*)((__bf16*)p.c + off) = v;
    } else {
      *(v4f*)((float*)p.c + off) = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K small-M GEMM (with a caller workspace). The small-M kernel above
// covers 32 columns per workgroup, so every workgroup re-reads all of A; for
// 64 x 7168 x 7168 that is twice the bytes of B. Here a workgroup owns a
// 64 x 128 tile (one weight block, so one B scale per group) and one of S
// contiguous K ranges: A is read N/128 times instead of N/32, and the S
// splits give about one workgroup per CU (never more, see splitk_splits).
// Per group the workgroup's A slab (64 x 128), B slab (128 x 128), the 64
// A-scales and the B scale all arrive by direct global -> LDS copies into a
// ring of three stages, two groups ahead; each of the 4 wavefronts multiplies
// its 32 columns and promotes like the large-tile kernel. The FP32 partial
// tile goes to workspace[split]; a second kernel sums the S partials in split
// order (deterministic) and writes C.
// ---------------------------------------------------------------------------
// s_waitcnt immediate that waits for vector-memory count <= n (0..63) and
// nothing else: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt at their maxima
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

constexpr int kSpM = 64;
constexpr int kSpN = 128;
constexpr int kSpWaves = 4;                     // one per 32 columns
constexpr int kSpLdsA = kSpM * 128;             // A slab of one group
constexpr int kSpLdsB = kSpN * 128;             // B slab of one group
constexpr int kSpStage = kSpLdsA + kSpLdsB + kSpM * 4 + 64 * 4;  // + A-scales, B scale
constexpr int kSpStages = 3;                    // copies run two groups ahead
constexpr int kSpWorkgroups = 256;              // CUs of the chip
constexpr int kSpCopies = 2 + 4 + 1 + 1;        // per thread per group: A, B, A-scales, B scale

__global__ __launch_bounds__(64 * kSpWaves) void gemm_splitk_kernel(GemmArgs p, float* __restrict__ ws,
                                                                    int S) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kSpStages * kSpStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lk = lane >> 4;
  const int G = p.K / kGroup;
  const int tiles_n = p.N / kSpN;
  const int nb = blockIdx.x % tiles_n;
  const int rest = blockIdx.x / tiles_n;
  const int split = rest % S;
  const int m0 = (rest / S) * kSpM;
  const int n0 = nb * kSpN;
  const int g_begin = (int)((int64_t)G * split / S);
  const int g_end = (int)((int64_t)G * (split + 1) / S);

  // Direct global -> LDS copies through buffer descriptors (rows past M read
  // as zeros: the row part of every offset is in the range-checked per-lane
  // offset, the group's advance in the scalar one). Slot t (16 bytes) of a
  // slab holds row t / 8, stored chunk t % 8, i.e. global chunk
  // (t % 8) ^ (row % 8); thread tid fills slots tid + 256 i.
  const int rows_a = min(kSpM, p.M - m0);
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(p.a + (int64_t)m0 * p.K, (uint32_t)rows_a * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(p.b + (int64_t)n0 * p.K, (uint32_t)kSpN * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t rsrc_sa = make_rsrc(p.sa + (int64_t)m0 * G, (uint32_t)rows_a * (uint32_t)G * 4);
  // the weight block's G scales; every lane copies the group's one scale (all
  // 64 slots of a stage hold it), which keeps it on the copy ring: a plain
  // load here would be a vector load whose use waits for every copy in flight
  const __amdgpu_buffer_rsrc_t rsrc_sb = make_rsrc(p.sb + (int64_t)(n0 / kGroup) * G, (uint32_t)G * 4);
  const int row0 = tid >> 3, lc0 = (tid & 7) ^ (row0 & 7);
  const uint32_t off0 = (uint32_t)row0 * (uint32_t)p.K + lc0 * 16;
  const uint32_t row_step = 32u * (uint32_t)p.K;  // slot + 256 = row + 32 (row % 8 kept)
  const uint32_t off_sa = (uint32_t)lane * (uint32_t)G * 4;
  auto issue = [&](int g, uint8_t* __restrict__ stage) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      load_lds(rsrc_a, stage + (i * 256 + wave * 64) * 16, 16, off0 + i * row_step, g * kGroup);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      load_lds(rsrc_b, stage + kSpLdsA + (i * 256 + wave * 64) * 16, 16, off0 + i * row_step, g * kGroup);
    // every wave copies the same 64 A-scales to the same place: uniform counts
    load_lds(rsrc_sa, stage + kSpLdsA + kSpLdsB, 4, off_sa, g * 4);
    load_lds(rsrc_sb, stage + kSpLdsA + kSpLdsB + kSpM * 4, 4, 0, g * 4);
  };

  const int lane_lo = lr * 128 + ((lk ^ (lr & 7)) << 4);
  const int lane_hi = lr * 128 + (((4 + lk) ^ (lr & 7)) << 4);
  auto load_frag = [&](const uint8_t* blk) {
    const uint4 lo = *(const uint4*)(blk + lane_lo);
    const uint4 hi = *(const uint4*)(blk + lane_hi);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  v4f acc[4][2];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = v4f{0.f, 0.f, 0.f, 0.f};

  // Multiply the group in `st` while the copy of a later group targets `nx`;
  // the restrict-qualified stages keep the compiler from waiting on that copy.
  auto compute = [&](const uint8_t* __restrict__ st, uint8_t* __restrict__ nx, int g, bool copy_next) {
    if (copy_next) issue(g + kSpStages - 1, nx);
    const float* ssa = (const float*)(st + kSpLdsA + kSpLdsB);
    const float sbv = ssa[kSpM];
    v8i bfr[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) bfr[jb] = load_frag(st + kSpLdsA + (wave * 32 + jb * 16) * 128);
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const v8i af = load_frag(st + ib * 16 * 128);
      const float sc = ssa[ib * 16 + lr] * sbv;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const v4f pp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bfr[jb], af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        acc[ib][jb][0] = __builtin_fmaf(pp[0], sc, acc[ib][jb][0]);
        acc[ib][jb][1] = __builtin_fmaf(pp[1], sc, acc[ib][jb][1]);
        acc[ib][jb][2] = __builtin_fmaf(pp[2], sc, acc[ib][jb][2]);
        acc[ib][jb][3] = __builtin_fmaf(pp[3], sc, acc[ib][jb][3]);
      }
    }
  };

  // prologue: the first kSpStages - 1 groups
#pragma unroll
  for (int d = 0; d < kSpStages - 1; ++d)
    if (g_begin + d < g_end) issue(g_begin + d, lds + d * kSpStage);
  for (int g = g_begin; g < g_end; ++g) {
    // this thread's copies of group g have landed once at most those of the
    // later groups already issued (up to kSpStages - 2 of them) are
    // outstanding: vector-memory loads complete in order
    const int later = min(kSpStages - 2, g_end - 1 - g);
    static_assert(kSpStages >= 2 && kSpStages <= 6, "wait table covers up to 4 later groups");
    switch (later) {
      case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(kSpCopies)); break;
      case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kSpCopies)); break;
      case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * kSpCopies)); break;
      default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * kSpCopies)); break;
    }
    // everyone's copies of g landed; everyone is done with g - 1. A bare
    // barrier: __syncthreads() would also wait for the copies still in flight.
    __builtin_amdgcn_s_barrier();
    const int st = (g - g_begin) % kSpStages;
    const int nx = (st + kSpStages - 1) % kSpStages;  // the stage g - 1 used
    compute(lds + st * kSpStage, lds + nx * kSpStage, g, g + kSpStages - 1 < g_end);
  }

  // partial tile -> workspace[split][m][n] (rows past M are not stored)
  float* wsp = ws + (int64_t)split * p.M * p.N;
  const int nw = n0 + wave * 32;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    const int gm = m0 + ib * 16 + lr;
    if (gm >= p.M) continue;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
      *(v4f*)(wsp + (int64_t)gm * p.N + nw + jb * 16 + 4 * lk) = acc[ib][jb];
  }
}

// C = sum over the S splits, in split order, then the output rounding. The
// partials are read kReduceBatch at a time, all loads of a batch in flight
// together: one dependent load per split made the kernel a chain of S memory
// latencies (about 4.5 us whatever the size).
constexpr int kReduceBatch = 16;

template <bool kBf16Out>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, void* c,
                                                            int64_t n4, int64_t MN, int S) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4 consecutive outputs
  if (i >= n4) return;
  const float* src = ws + 4 * i;
  v4f sum = *(const v4f*)src;
  for (int s0 = 1; s0 < S; s0 += kReduceBatch) {
    v4f part[kReduceBatch];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u)
      if (s0 + u < S) part[u] = *(const v4f*)(src + (int64_t)(s0 + u) * MN);
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u)
      if (s0 + u < S) sum += part[u];
  }
  if constexpr (kBf16Out) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    *(bf16x4*)((__bf16*)c + 4 * i) = bf16x4{(__bf16)sum[0], (__bf16)sum[1], (__bf16)sum[2], (__bf16)sum[3]};
  } else {
    *(v4f*)((float*)c + 4 * i) = sum;
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool kGrouped, bool kRowB>
static hipError_t launch_cfg(GemmArgs args, bool bf16_out, int m_tiles, hipStream_t stream) {
  using Cfg = TileCfg<BM, BN, WAVES_M, WAVES_N, kRowB>;
  args.n_tiles = m_tiles * ((args.N + BN - 1) / BN);
  const dim3 block(Cfg::kThreads);
  // Dense tail: when the tiles fill their last wave of workgroups (one per
  // CU) at most half, the last c tile columns, enough to hold that wave,
  // go in BM x BN/2 tiles instead.
  const int rem = args.n_tiles % kCus;
  if constexpr (!kGrouped && !kRowB) {
    if (args.n_tiles > kCus && rem > 0 && rem <= kCus / 2) {
    const int n_tiles_n = (args.N + BN - 1) / BN;
    const int c = (rem + m_tiles - 1) / m_tiles;  // tile columns to split
    if (c < n_tiles_n) {
      args.n_col_main = (n_tiles_n - c) * BN;
      args.n_big = m_tiles * (n_tiles_n - c);
      const int n_half = m_tiles * ((args.N - args.n_col_main) / (BN / 2));
      const dim3 grid((unsigned)(args.n_big + n_half));
      if (bf16_out)
        hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WAVES_M, WAVES_N, true, kGrouped, kRowB, true>),
                           grid, block, 0, stream, args);
      else
        hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WAVES_M, WAVES_N, false, kGrouped, kRowB, true>),
                           grid, block, 0, stream, args);
      return hipGetLastError();
    }
    }
  }
  const dim3 grid((unsigned)args.n_tiles);
  if (bf16_out) {
    hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WAVES_M, WAVES_N, true, kGrouped, kRowB, false>),
                       grid, block, 0, stream, args);
  } else {
    hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WAVES_M, WAVES_N, false, kGrouped, kRowB, false>),
                       grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

// Workgroups of the 256 x 256 kernel below which the small-M kernel is used:
// fewer big tiles than this leave most of the 256 CUs idle.
constexpr int64_t kSmallTileCount = 128;

template <bool kRowB>
static hipError_t launch_dense(GemmArgs args, bool bf16_out, hipStream_t stream) {
  const int64_t M = args.M, N = args.N;
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles < kSmallTileCount) {
    const dim3 grid((unsigned)(((M + kSkM - 1) / kSkM) * (N / kSkN)));
    if (bf16_out)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, kRowB>), grid, dim3(64 * kSkWaves), 0, stream, args);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<false, kRowB>), grid, dim3(64 * kSkWaves), 0, stream, args);
    return hipGetLastError();
  }
  return launch_cfg<256, 256, 2, 4, false, kRowB>(args, bf16_out, (int)((M + 255) / 256), stream);
}

hipError_t launch_gemm_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                   const float* sb, void* c, bool bf16_out, int64_t M, int64_t N,
                                   int64_t K, hipStream_t stream) {
  return launch_dense<false>(GemmArgs{a, sa, b, sb, c, nullptr, (int)M, (int)N, (int)K, 1, 0},
                             bf16_out, stream);
}

// Split-K plan for small-M shapes (those the small-M kernel would take): S
// splits of the K groups; 0 when the shape does not take the split-K path.
int splitk_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  // with fewer than 16 groups the splits hold one or two groups each and the
  // second launch costs more than the split saves (256 x 256 x 1024: 7.9 us
  // split, 6.1 us in one launch of the small-M kernel)
  if (big_tiles >= kSmallTileCount || K < 16 * kGroup) return 0;
  const int64_t tiles = ((M + kSpM - 1) / kSpM) * (N / kSpN);
  const int64_t G = K / kGroup;
  // at most one workgroup per CU: a deep copy ring leaves room for only one,
  // and a second round of workgroups would double the time
  int64_t S = kSpWorkgroups / tiles;
  S = S < G ? S : G;
  return S >= 2 ? (int)S : 0;
}

int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = splitk_splits(M, N, K);
  return S ? (int64_t)S * M * N * 4 : 0;
}

hipError_t launch_gemm_blockscaled_ws(const uint8_t* a, const float* sa, const uint8_t* b,
                                      const float* sb, void* c, bool bf16_out, int64_t M,
                                      int64_t N, int64_t K, float* ws, hipStream_t stream) {
  const int S = splitk_splits(M, N, K);
  GemmArgs args{a, sa, b, sb, c, nullptr, (int)M, (int)N, (int)K, 1, 0};
  if (!S) return launch_dense<false>(args, bf16_out, stream);
  const int64_t tiles = ((M + kSpM - 1) / kSpM) * (N / kSpN);
  hipLaunchKernelGGL(gemm_splitk_kernel, dim3((unsigned)(tiles * S)), dim3(64 * kSpWaves), 0, stream,
                     args, ws, S);
  const int64_t n4 = M * N / 4;
  const dim3 grid((unsigned)((n4 + 255) / 256));
  if (bf16_out)
    hipLaunchKernelGGL(splitk_reduce_kernel<true>, grid, dim3(256), 0, stream, ws, c, n4, M * N, S);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<false>, grid, dim3(256), 0, stream, ws, c, n4, M * N, S);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K partials in library-owned device memory, for callers that cannot
// allocate: a file-scope array, one copy per GPU the library runs on, held
// until the process ends. Host code never passes the array's name to a
// kernel (in host code it is only a stand-in for the symbol): the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
// ---------------------------------------------------------------------------
constexpr int64_t kStaticScratchBytes = int64_t(8) << 20;
static __device__ __align__(256) float scratch[kStaticScratchBytes / 4];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<float*> g_scratch_ptr[kScratchDevices];
}  // namespace

int64_t static_scratch_bytes() { return kStaticScratchBytes; }

// The current device's copy of `scratch`; resolved on the first call per device.
static hipError_t scratch_ptr(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  float* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr = (float*)q;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // same value from any racing thread
  }
  *out = ptr;
  return hipSuccess;
}

// fp8_gemm_blockscaled_ws with the partials in `scratch` (the caller has
// checked that splitk_workspace_bytes(M, N, K) <= kStaticScratchBytes).
hipError_t launch_gemm_blockscaled_static(const uint8_t* a, const float* sa, const uint8_t* b,
                                          const float* sb, void* c, bool bf16_out, int64_t M,
                                          int64_t N, int64_t K, hipStream_t stream) {
  float* ws = nullptr;
  if (splitk_workspace_bytes(M, N, K) > 0) {
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return e;
  }
  return launch_gemm_blockscaled_ws(a, sa, b, sb, c, bf16_out, M, N, K, ws, stream);
}

hipError_t launch_gemm_rowscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                 const float* sb_rows, void* c, bool bf16_out, int64_t M, int64_t N,
                                 int64_t K, hipStream_t stream) {
  return launch_dense<true>(GemmArgs{a, sa, b, sb_rows, c, nullptr, (int)M, (int)N, (int)K, 1, 0},
                            bf16_out, stream);
}

hipError_t launch_gemm_grouped(const uint8_t* a, const float* sa, const uint8_t* b,
                               const float* sb, void* c, bool bf16_out, const int32_t* m_offsets,
                               int64_t G, int64_t M_total, int64_t N, int64_t K,
                               hipStream_t stream) {
  GemmArgs args{a, sa, b, sb, c, m_offsets, (int)M_total, (int)N, (int)K, (int)G, 0};
  // upper bound on sum_e ceil(rows_e / 256) for rows_e multiples of 128
  const int64_t m_tiles = (M_total / 128 + G + 1) / 2;
  return launch_cfg<256, 256, 2, 4, true, false>(args, bf16_out, (int)m_tiles, stream);
}

}  // namespace fp8q
