// K3 / K5: absorbed MLA attention over the paged bf16 latent cache (decode
// split over the cache, and causal chunked prefill), and K4: the merge of
// decode splits.
//
// What one row computes ("AI decoupled RoPE MLA", decoupled-RoPE score
// equation, with one scale on the summed score; "Multi-Head Latent
// Attention", "Why this matters on a GPU": softmax and the weighted sum stay):
//   s_t  = scale * Q_lat[row] . cache[t]           (576 = 512 + 64 wide:
//          q~ . c_t  +  R_m q^R . R_t k^R_t, both halves in one dot product)
//   obar = sum_t softmax(s)_t * cache[t][0 : d_c]  (V = first d_c columns)
//
// Every head of a query reads the same cache row ("Latent Attention Meets
// RoPE": one latent and one shared position key per token), so a workgroup
// takes 32*HG rows (heads, or (query, head) pairs in prefill) against one
// stream of cache tiles, and both products are dense MFMA contractions:
//   S^T[token, row]  = K[token, 0:D]  . Q^T[0:D, row]    (v_mfma 32x32x16 bf16)
//   O^T[c, row]     += V^T[c, token] . P^T[token, row]
// Layout per workgroup:
//   * Q for a wave's 32 rows: most k-steps in VGPRs, the rest in LDS;
//   * O in float32 accumulators (AGPRs).  With four head groups the P.V
//     product is split by columns: each wave accumulates d_c/4 columns of
//     all rows, P is exchanged through LDS once per tile, and one V^T
//     transpose read serves four head groups;
//   * the cache streams HBM -> LDS by 16-byte buffer-load DMA into a ring of
//     three 32-row tiles, read by every wave; 16-byte chunks are
//     XOR-swizzled so every K read phase and V^T transpose half-wave hits
//     distinct banks;
//   * V^T fragments come from the same tile with ds_read_tr16_b64, which
//     turns four 8-byte row pieces into one token-contiguous column piece;
//   * softmax in base 2 without rescaling O inside the loop: each row's
//     reference max is fixed at its first visible key and P = 2^(s - m_ref)
//     may grow; a lane whose sum of P ends too large makes the workgroup redo
//     the split exactly in two passes (true max, then accumulate).  The same
//     data always takes the same path, so the result is deterministic.  (A
//     VALU rescale of the 256 accumulator registers would force them out of
//     AGPRs and spill.)
// Tokens past the end of a sequence are masked; their LDS rows are filled
// from the last valid row of the tile, so garbage or NaN in unused page
// slots never reaches the accumulators.
//
// Precision.  obar and the split partials are float32 (normalised rows).  By
// default q_lat and the softmax weights P fed to P.V are bf16.  The float32
// working precision (F32W, the small shape only) takes a float32 q_lat and
// feeds both q~ and P to their contractions as two-term bf16 splits
// (x = hi + lo, hi = bf16(x), lo = bf16(x - hi)), so neither is rounded to
// bf16 once; the contractions then take twice the MFMAs.
#include <cfloat>
#include <type_traits>

#include "common.hpp"
#include "decode_items.hpp"

namespace mla {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kOverflowMax = 18446744073709551616.0f;  // 2^64: a lane's sum of P beyond it redoes the split
// Word 3 of a raw (untyped) buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle, no index/thread-id addressing.
constexpr int kBufferWord3 = 0x00020000;

// XOR swizzle of row r: bit 1 of the row to bit 2, bits 2-3 to bits 0-1 (a
// function of r mod 16).  With 64 four-byte banks and 1152-byte rows (odd rows
// start half way round the banks), it puts every 16-lane phase of a K read
// (16 rows, one chunk each) and every half-wave of a V transpose read (4 rows
// x 4 chunks x 8 bytes in two pieces) on distinct banks.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Physical 16-byte chunk slot of logical chunk j in LDS row r.  Full groups
// of 8 chunks are XOR-swizzled with swz(r); a trailing group of 4 (when the
// row is not a multiple of 8 chunks) with swz(r) & 3.  An involution: the
// same function maps physical slots back to logical chunks.
template <int D>
__device__ __forceinline__ int phys_chunk(int r, int j) {
  constexpr int CHF = (D / 8 / 8) * 8;
  if constexpr (CHF == D / 8) return j ^ swz(r);  // every chunk is in a full group: no branch
  return j < CHF ? (j ^ swz(r)) : (j ^ (swz(r) & 3));
}


struct PrefillBlock {
  int b, rb;
  bool ok;
};

// Prefill row blocks: sequence b has ceil(n_q(b) * H / rows) blocks of
// `rows` consecutive (query, head) rows; blocks are issued last-first so
// the long causal rows start first.
__device__ PrefillBlock find_prefill_block(const AttnParams& p, int64_t blk, int rows) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int b = b0 + lane;
    int nb = 0;
    if (b < p.batch) {
      const int nq = p.cu_q[b + 1] - p.cu_q[b];
      nb = nq > 0 ? (nq * p.n_heads + rows - 1) / rows : 0;
    }
    const int incl = wave_incl_scan(nb);
    const int lo = base + incl - nb;
    const bool hit = nb > 0 && blk >= lo && blk < lo + nb;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __ffsll(static_cast<long long>(mask)) - 1;
      PrefillBlock r{b0 + src, static_cast<int>(blk) - __shfl(lo, src, 64), true};
      return r;
    }
    base += __shfl(incl, 63, 64);
  }
  PrefillBlock none{0, 0, false};
  return none;
}

// Tile DMA: TROWS consecutive cache rows of D bf16 (starting at `src`) go
// into an LDS buffer by 16-byte buffer-load DMA.  LDS chunk slot sl of
// tile row r holds logical chunk phys_chunk(r, sl) of that row.  Rows go in
// groups of RG rows = 576 chunks = 9 wave instructions; a wave takes whole
// groups (when there are fewer groups than waves, the first NG waves take
// one each), so a lane's (row-in-group, slot) pairs depend only on the lane
// and the LDS destination of every instruction is wave-uniform.  Rows
// >= valid_rows read row valid_rows - 1.  Each issuing wave has
// dma_loads<D, NW, TROWS>() loads in flight per tile.
template <int D, int TROWS>
constexpr int dma_groups() { return TROWS / (576 / (D / 8)); }
template <int D, int NW, int TROWS>
constexpr int dma_loads() { return 9 * (dma_groups<D, TROWS>() >= NW ? dma_groups<D, TROWS>() / NW : 1); }

// One tile's DMA: the source resource and valid rows prepared once, then
// issued as N 1 KiB wave instructions.  CPOL is the loads' cache policy.
template <int D, int NW, int TROWS, int CPOL>
struct TileDma {
  static constexpr int CH = D / 8;
  static constexpr int ROWB = D * 2;
  static constexpr int RG = 576 / CH;
  static constexpr int NG = dma_groups<D, TROWS>();
  static constexpr int GPW = NG >= NW ? NG / NW : 1;
  static constexpr int N = 9 * GPW;  // instructions per issuing wave
  static_assert(RG * CH == 576 && TROWS % RG == 0 && (NG < NW || NG % NW == 0), "tile must split into row groups");
  __amdgpu_buffer_rsrc_t rsrc;
  lds_char_t* lds_buf;  // LDS address of the tile buffer
  int valid_rows;
  bool active;  // wave-uniform: this wave has instructions to issue for this tile

  // A raw buffer resource over the tile: the DMA goes through the buffer
  // path, whose completion the compiler tracks on the vector-memory counter
  // alone, so LDS reads in flight keep exact wait counts.  Offsets past the
  // tile would read zeros; none are formed.
  __device__ __forceinline__ TileDma(char* dst, const char* src, int valid, bool on, int wave)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), 0, TROWS * ROWB, kBufferWord3)),
        lds_buf(reinterpret_cast<lds_char_t*>(reinterpret_cast<uintptr_t>(dst))), valid_rows(valid), active(on && (NG >= NW || wave < NG)) {}

  // Byte offset in the tile of a lane's 16 bytes in instruction i (0 <= i <
  // N, a compile-time constant at every call site) of wave `wave`, for a
  // tile whose rows >= valid repeat row valid - 1.
  __device__ __forceinline__ static uint32_t offset(int i, int lane, int wave, int valid) {
    const int gg = i / 9, kk = i % 9;
    const int g = NG >= NW ? wave * GPW + gg : wave;
    const int c = kk * 64 + lane;
    const int rig = c / CH;
    const int r = g * RG + rig;
    const int j = phys_chunk<D>(r, c - rig * CH);
    const int rs = r < valid ? r : valid - 1;
    return static_cast<uint32_t>(rs * ROWB + j * 16);
  }
  // A full tile's offsets depend on the lane and the wave only, so they are
  // computed once per kernel and kept two 16-bit values to a register; the
  // division and swizzle behind them cost far more than the DMA issue.
  static_assert(TROWS * ROWB <= 65536, "tile offsets must fit 16 bits");
  struct Full {
    uint32_t v[(N + 1) / 2];
  };
  __device__ __forceinline__ static Full full_offsets(int lane, int wave) {
    Full f;
#pragma unroll
    for (int i = 0; i < N; i += 2)
      f.v[i / 2] = offset(i, lane, wave, TROWS) | (i + 1 < N ? offset(i + 1, lane, wave, TROWS) << 16 : 0u);
    return f;
  }
  __device__ __forceinline__ void issue_at(int i, int wave, uint32_t off) const {
    const int gg = i / 9, kk = i % 9;
    const int g = NG >= NW ? wave * GPW + gg : wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_buf + g * RG * ROWB + kk * 1024, 16, off, 0, 0,
                                             CPOL);
  }
  // A full tile (valid_rows == TROWS) from the precomputed offsets.
  __device__ __forceinline__ void issue_full(int wave, const Full& f) const {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < N; ++i) issue_at(i, wave, (f.v[i / 2] >> (16 * (i % 2))) & 0xffffu);
  }
  __device__ __forceinline__ void issue_all(int lane, int wave, const Full& f) const {
    if (!active) return;
    if (valid_rows == TROWS) {
      issue_full(wave, f);
    } else {
      // the last tile of a sequence: offsets recomputed from an opaque lane
      // id (not hoisted into more registers)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        issue_at(i, wave, offset(i, ln, wave, valid_rows));
      }
    }
  }
};

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding and does not wait on the other counters (gfx9 encoding).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// S += K . Q^T on VGPR accumulators (v_mfma_f32_32x32x16_bf16, 16 floats a
// lane).  Written as inline asm so that the score accumulators live in VGPRs
// while the output accumulators hold the AGPRs (the compiler otherwise puts
// both in AGPRs and spills).  The first step of an accumulator uses an inline
// zero for srcC, so no VALU write feeds an MFMA.
__device__ __forceinline__ void mfma_qk_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// Wait states between the last score MFMAs and the VALU reads of their
// results (the hazard recognizer does not see inside inline asm).
__device__ __forceinline__ void mfma_qk_drain(f32x16& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}

// MFMA 32x32x16 lane layouts used below (lane l, r = l % 32, h = l / 32):
//   A[i][k]: row i = r, k = 8h .. 8h+7;   B[k][j]: column j = r, k = 8h .. 8h+7;
//   D[i][j]: column j = r, rows i = 8g + 4h + e in register 4g + e (g, e < 4).
template <int DC, int DR, int HG, int TW, bool PREFILL, bool F32W>
__global__ void __launch_bounds__(64 * HG * TW, 1) attn_bf16_kernel(AttnParams p) {
  constexpr int D = DC + DR;
  constexpr int ROWB = D * 2;       // bytes per cache row
  constexpr int NT = 64 * HG * TW;
  constexpr int NW = NT / 64;       // waves
  constexpr int ROWS = 32 * HG;
  constexpr int KS = D / 16;        // 16-wide k steps of the score contraction
  // Four head groups of one token lane split P.V by columns of O: each wave
  // accumulates all 128 rows over d_c/4 columns, so one V^T transpose read
  // serves four head groups (a quarter of the transpose traffic), and P
  // (32 tokens x 128 rows, bf16) is exchanged through LDS once per tile.
  constexpr bool DSPLIT = HG == 4 && TW == 1;
  // Q k-steps kept in LDS: the position part, plus (at d_c = 512) content
  // k-steps, which keeps the page loop within the register file (two fewer
  // with the column split, whose P buffer takes their LDS).
  constexpr int KSL = DR / 16 + (DC >= 512 ? (DSPLIT ? 6 : 8) : 0);
  constexpr int KSQ = KS - KSL;     // Q k-steps kept in VGPRs
  constexpr int QCH = KSL * 2;      // 16-byte chunks per row of the LDS part of Q
  static_assert(DR % 16 == 0 && QCH % 4 == 0, "LDS part of Q must swizzle within its row");
  constexpr int CB = DC / 32;       // 32-wide column blocks of O
  constexpr int CBW = DSPLIT ? CB / 4 : CB;  // column blocks a wave accumulates
  static_assert(!DSPLIT || CBW % 2 == 0, "a wave's columns must cover whole swizzle groups");
  constexpr int PAGE_BYTES = kPage * D * 2;
  // LDS tiles of TROWS cache rows (32 per wave token lane), in a ring of three:
  // one being read, two in flight.
  constexpr int TROWS = 32 * TW;
  constexpr int TILE = TROWS * D * 2;
  constexpr int G = dma_loads<D, 64 * HG * TW / 64, TROWS>();
  static_assert(D % 32 == 0 && DC % 32 == 0, "dims");
  static_assert(TW == 1 || HG <= 2, "two token lanes need half the waves' registers");
  __shared__ __attribute__((aligned(16))) char lds0[TILE];
  __shared__ __attribute__((aligned(16))) char lds1[TILE];
  __shared__ __attribute__((aligned(16))) char lds2[TILE];
  __shared__ bf16x8 ldsq[(F32W ? 2 : 1) * ROWS * QCH];
  // P^T of a tile for the column split: entry (kp * 2 + h) * ROWS + row holds
  // row's P at the 8 tokens that half h of k-step kp covers (with F32W, the
  // lo terms follow at 4 * ROWS)
  __shared__ bf16x8 ldsp[DSPLIT ? (F32W ? 8 : 4) * ROWS : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave % HG;
  const int tw = wave / HG;
  const int r32 = lane & 31, h2 = lane >> 5;
  const int H = p.n_heads;

  // ---- which rows and which keys.  Everything here is wave-uniform except
  // the row a lane serves: lanes l and l ^ 32 serve local row lrow of the
  // workgroup's ROWS rows, global row row_base + lrow, valid when lrow <
  // row_count.  Row addresses are recomputed where needed instead of being
  // held across the page loop.
  int b, page_begin, page_end, key_end, row_count;
  int64_t row_base;
  int limit;
  bool final_out = true;
  int slot = 0;
  const int lrow = hg * 32 + r32;
  if constexpr (PREFILL) {
    const int64_t wg = xcd_local(blockIdx.x, gridDim.x);
    const PrefillBlock pb = find_prefill_block(p, p.n_blocks - 1 - wg, ROWS);
    if (!pb.ok) return;
    b = __builtin_amdgcn_readfirstlane(pb.b);
    const int nq = __builtin_amdgcn_readfirstlane(p.cu_q[b + 1] - p.cu_q[b]);
    const int q0 = __builtin_amdgcn_readfirstlane(p.q_start[b]);
    const int r0 = __builtin_amdgcn_readfirstlane(pb.rb) * ROWS;
    const int last_q = min(nq - 1, (r0 + ROWS - 1) / H);
    key_end = __builtin_amdgcn_readfirstlane(q0 + last_q + 1);
    page_begin = 0;
    page_end = (key_end + kPage - 1) / kPage;
    row_base = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(p.cu_q[b])) * H + r0;
    row_count = nq * H - r0;
    limit = lrow < row_count ? q0 + (r0 + lrow) / H + 1 : 0;
  } else {
    const int64_t wg = xcd_local(blockIdx.x, gridDim.x);
    const int64_t item = wg / p.n_head_chunks;
    const int hc = static_cast<int>(wg % p.n_head_chunks);
    const DecodeItem it = find_decode_item(p, item);
    if (!it.ok || it.slot >= p.n_items) return;
    // the item is wave-uniform: keep it in scalar registers
    b = __builtin_amdgcn_readfirstlane(it.b);
    key_end = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
    const int pages = (key_end + kPage - 1) / kPage;
    page_begin = __builtin_amdgcn_readfirstlane(it.s) * p.split_pages;
    page_end = min(pages, page_begin + p.split_pages);
    final_out = !p.all_partials && __builtin_amdgcn_readfirstlane(it.n_s) == 1;
    slot = __builtin_amdgcn_readfirstlane(it.slot);
    row_base = static_cast<int64_t>(b) * H + hc * ROWS;
    row_count = H - hc * ROWS;
    limit = key_end;
  }
  if (b >= p.num_seqs) return;
  // wave-uniform bound on the visible keys of this wave's rows (of the whole
  // workgroup with the column split, whose tiles every wave must take)
  int lim_max = limit;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) lim_max = max(lim_max, __shfl_xor(lim_max, m, 64));
  lim_max = __builtin_amdgcn_readfirstlane(DSPLIT ? key_end : lim_max);
  // wave-uniform lower bound: sub-blocks entirely below it need no mask
  int lim_min = lrow < row_count ? limit : INT32_MAX;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, m, 64));
  lim_min = __builtin_amdgcn_readfirstlane(lim_min);

  // ---- Q fragments (MFMA B operand: row = r32, d = ks*16 + 8*h2 .. +7).
  // A float32 q_lat is split into hi = bf16(q) and lo = bf16(q - hi); the
  // score then takes both terms (K.hi + K.lo), so q~ enters at ~16 bits.
  // The first KSQ k-steps stay in VGPRs; the last KSL go to LDS, where each
  // lane keeps exactly the fragments it will read back (no sharing, so no
  // barrier), XOR-swizzled like the cache tiles.
  bf16x8 qf[KSQ];
  bf16x8 qlo[F32W ? KSQ : 1];
  // this lane's LDS home of a fragment of k-step ks; lr, lh are the lane's r32, h2.
  // Rows of a multiple of 8 chunks take the cache tiles' swizzle; other rows
  // (a stride of 16 banks mod 64) XOR with bits 2-3 of the row.  Either way
  // the 16 rows of every read phase land on distinct banks.
  auto q_slot = [&](int term, int ks, int lr, int lh) -> bf16x8* {
    const int row = hg * 32 + lr;
    const int ch = (ks - KSQ) * 2 + lh;
    const int x = QCH % 8 == 0 ? (swz(row) & 7) : ((row >> 2) & 3);
    return &ldsq[(term * ROWS + row) * QCH + (ch ^ x)];
  };
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 hi8, lo8;
    if constexpr (F32W) {
      const float* qlat = static_cast<const float*>(p.q_lat);
      bf16_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = lrow < row_count ? qlat[(row_base + lrow) * D + ks * 16 + h2 * 8 + e] : 0.f;
        hi[e] = f32_to_bf16_finite(x);
        lo[e] = f32_to_bf16_finite(x - bf16_to_f32(hi[e]));
      }
      __builtin_memcpy(&hi8, hi, 16);
      __builtin_memcpy(&lo8, lo, 16);
    } else {
      const bf16_t* qlat = static_cast<const bf16_t*>(p.q_lat);
      hi8 = lrow < row_count ? *reinterpret_cast<const bf16x8*>(qlat + (row_base + lrow) * D + ks * 16 + h2 * 8)
                             : bf16x8{};
    }
    if (ks < KSQ) {
      qf[ks < KSQ ? ks : 0] = hi8;
      if constexpr (F32W) qlo[ks < KSQ ? ks : 0] = lo8;
    } else {
      *q_slot(0, ks, r32, h2) = hi8;
      if constexpr (F32W) *q_slot(1, ks, r32, h2) = lo8;
    }
  }

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  const char* cache = static_cast<const char*>(p.cache);
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  // Page ids of the split, 64 at a time: lane j holds page (base + j); a
  // tile reads its id with readlane, so the loop issues no other vector loads.
  auto load_ids = [&](int first_pg) -> int {
    const int pg = first_pg + lane;
    int id = (pg < page_end && pg < p.max_pages) ? bt[pg] : 0;
    return (id < 0 || id >= p.num_pages) ? 0 : id;
  };
  auto page_ptr = [&](int ids, int pg) -> const char* {
    const int id = __builtin_amdgcn_readlane(ids, (pg - page_begin) & 63);
    return cache + static_cast<int64_t>(id) * PAGE_BYTES;
  };

  constexpr int CHF8 = (D / 8 / 8) * 8;  // chunks in full swizzle groups

  // tiles covering the split's keys [page_begin * 64, min(page_end * 64, key_end))
  const int key_hi = min(page_end * kPage, key_end);
  const int ntile = key_hi > page_begin * kPage ? (key_hi - page_begin * kPage + TROWS - 1) / TROWS : 0;

  // One pass over the split's pages.  MODE 0: the reference max of a row is
  // fixed at its first visible key and P = 2^(s - m_ref) may grow; a lane
  // whose sum of P ends above kOverflowMax (or not finite) sets `overflow`.
  // Below that bound every P and every partial of O stay far inside the
  // float32 and bf16 ranges, so the pass is exact.  MODE 1: running max only
  // (no PV).  MODE 2: P = 2^(s - m) with the true max m from a MODE 1 pass.
  // O is never rescaled inside the loop.
  // Per-lane LDS byte offsets inside a 32-row sub-block, the same for every
  // tile: swizzle groups, token halves and column blocks enter as
  // immediates (rows 16 apart share a swizzle).
  // K (A operand) of k-step ks: token row r32, chunk 2*ks + h2; group ks/4
  int k_off[4], k_tail[2];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) k_off[kq] = r32 * ROWB + phys_chunk<D>(r32, 2 * kq + h2) * 16;
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) k_tail[kq] = r32 * ROWB + phys_chunk<D>(r32, CHF8 + 2 * kq + h2) * 16;
  // V^T (A operand) of k-step kp, column block cb, transpose read s:
  // supplier lane 16g + 4k + q reads token row 16kp + 8s + 4(g/2) + k,
  // columns cb*32 + 16(g%2) + 4q .. +3; the result gives lane l the
  // column cb*32 + l%32 at tokens 16kp + 8s + 4h + 0..3, the order in
  // which the lane holds P.
  int v_off[2][2];
  {
    const int vg = lane >> 4, vk = (lane >> 2) & 3, vq = lane & 3;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int vrow = 8 * s + 4 * (vg >> 1) + vk;
#pragma unroll
      for (int co = 0; co < 2; ++co)
        v_off[s][co] = vrow * ROWB + phys_chunk<D>(vrow, 4 * co + 2 * (vg & 1) + (vq >> 1)) * 16 + (vq & 1) * 8;
    }
  }

  // Decode reads every cache row once, in one workgroup: nt marks its lines for
  // early eviction (2-3% faster at 64 x 4096).  Prefill re-reads a sequence's
  // rows in every query block, so its loads keep the default policy.
  using Dma = TileDma<D, NW, TROWS, PREFILL ? 0 : kCpolNt>;
  const typename Dma::Full dma_full = Dma::full_offsets(lane, wave);
  auto run_pass = [&](auto mode_tag) -> bool {
    constexpr int MODE = decltype(mode_tag)::value;
    bool overflow = false;
    int ids = load_ids(page_begin);
    // source of tile h: page page_begin + h*TROWS/64, from row (h*TROWS) % 64
    auto tile_dma = [&](int h, char* dst) -> Dma {
      const int rel = h * TROWS;
      const int pg = page_begin + rel / kPage;
      if (rel % kPage == 0 && ((pg - page_begin) & 63) == 0 && pg != page_begin) ids = load_ids(pg);
      const int t0 = page_begin * kPage + rel;
      return Dma(dst, page_ptr(ids, pg) + (rel % kPage) * ROWB, min(TROWS, key_end - t0), true, wave);
    };
    if (ntile > 0) tile_dma(0, lds0).issue_all(lane, wave, dma_full);
    if (ntile > 1) tile_dma(1, lds1).issue_all(lane, wave, dma_full);
    // One tile: wait for `cur` (the next tile's DMA stays in flight), make it
    // visible to all waves, start the DMA two tiles ahead into `nx2` (the
    // buffer every wave finished reading one step ago), compute on `cur`.  The three buffers are distinct LDS objects, so the compiler can
    // see that the DMAs in flight never alias the reads.
    auto tile = [&](int it, char* cur, char* nx2) {
      if (it + 1 < ntile)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(G));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      // A bare barrier: __syncthreads() would also drain the DMA still in
      // flight.  Every LDS read of the previous tile has been consumed by an
      // MFMA by now; the memory clobber keeps this tile's reads below it.
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // The DMA two tiles ahead.  The CU's address unit takes a 1 KiB
      // instruction about every 16 cycles and stalls the issuing wave while
      // busy, so the waves take turns: wave w issues its burst at score
      // k-step w * KS / NW, while the others keep their MFMAs going.
      const bool dma_on = it + 2 < ntile;
      const Dma dma = tile_dma(dma_on ? it + 2 : ntile - 1, nx2);  // issued only when dma_on
      constexpr int DMA_KSTEP = KS / NW;
      // a sequence's last, partial tile takes the slow offsets, in one burst here
      const bool dma_turn = dma_on && dma.valid_rows == TROWS;
      if (dma_on && !dma_turn) dma.issue_all(lane, wave, dma_full);
      const int sb = TW == 1 ? 0 : tw;  // this wave's 32-row sub-block of the tile
      const char* buf = cur + sb * 32 * ROWB;
      const int t0 = page_begin * kPage + it * TROWS + sb * 32;
      [&] {
        // skip sub-blocks no row of this wave can see (wave-uniform)
        if (t0 >= lim_max) {
          if (dma_turn) dma.issue_full(wave, dma_full);
          return;
        }
        const int lr = lane & 31, lh = lane >> 5;
        // ---- S^T = K . Q^T over D, one accumulator (dependent accumulation
        // issues back to back at full rate)
        f32x16 sacc;
        // K fragments run KPF steps ahead of the MFMAs that consume them.
        constexpr int KPF = 8;
        bf16x8 ka[KS];
        bf16x8 qr[KS], qrlo[F32W ? KS : 1];
        auto load_k = [&](int ks) {
          const char* a = 2 * ks < CHF8 ? buf + k_off[ks & 3] + (ks / 4) * 128 : buf + k_tail[(ks - CHF8 / 2) & 1];
          ka[ks] = *reinterpret_cast<const bf16x8*>(a);
          if (ks >= KSQ) {
            qr[ks] = *q_slot(0, ks, lr, lh);
            if constexpr (F32W) qrlo[ks] = *q_slot(1, ks, lr, lh);
          }
        };
#pragma unroll
        for (int ks = 0; ks < KPF; ++ks) load_k(ks);
        asm volatile("s_nop 1" ::: "memory");
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + KPF < KS) load_k(ks + KPF);
          if (ks % DMA_KSTEP == 0 && ks / DMA_KSTEP < NW && ks / DMA_KSTEP == wave && dma_turn)
            dma.issue_full(wave, dma_full);
          const bf16x8& qb = ks < KSQ ? qf[ks < KSQ ? ks : 0] : qr[ks];
          if (ks == 0)
            mfma_qk_first(sacc, ka[ks], qb);
          else
            mfma_qk(sacc, ka[ks], qb);
          if constexpr (F32W) mfma_qk(sacc, ka[ks], ks < KSQ ? qlo[ks < KSQ ? ks : 0] : qrlo[F32W ? ks : 0]);
          __builtin_amdgcn_sched_barrier(0);  // keep the K reads of step ks + KPF above the MFMA of step ks
        }
        mfma_qk_drain(sacc);
        // ---- reference max.  Raw scores stay unscaled; the scale (times log2 e)
        // is folded into the exponent's FMA.  Lane (row lr, half lh) holds
        // tokens 8g + 4lh + e at register 4g + e.  Only sub-blocks that cross a
        // row's last visible key are masked.  The row max (with one swap with
        // lane l ^ 32) is needed only while a row has no reference yet (its
        // first visible sub-block) and in the max-only pass.
        float sv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
        const bool partial = t0 + 32 > lim_min;
        if (partial) {
          float ninf = -INFINITY;  // materialised here, not held across the loop
          asm volatile("" : "+v"(ninf));
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = t0 + 8 * g + 4 * lh + e;
              if (t >= (PREFILL ? limit : key_end)) sv[4 * g + e] = ninf;
            }
        }
        const bool need_ref = MODE == 1 || __ballot(m_run == -INFINITY) != 0;
        if (need_ref) {
          float lmx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) lmx = fmaxf(lmx, sv[i]);
          lmx *= p.scale_log2;  // this lane's max (scale > 0 keeps the order)
          const float m = pair32_max(lmx);
          if constexpr (MODE == 1)
            m_run = fmaxf(m_run, m);
          else if (m_run == -INFINITY)
            m_run = m;  // O and l are still zero: exact
        }
        if constexpr (MODE == 1) return;
        // ---- P = 2^(scale*log2e*s - m) rounded to bf16 (hardware RNE, two at a
        // time); registers 8kp .. 8kp+7 are the B operand of k-step kp.
        bf16x8 pb[2], pl[F32W ? 2 : 1];
        // a row still without a reference has only masked (-inf) scores here,
        // which give 0 against any finite reference
        const float m_use = __builtin_fmaxf(m_run, -FLT_MAX);
        // P of k-step kp into pb[kp] (and its lo term into pl[kp]); returns
        // the float32 sum of the unrounded weights
        auto p_half = [&](int kp) -> float {
          float pf[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[8 * kp + e], p.scale_log2, -m_use));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x2 pair = __builtin_convertvector((f32x2){pf[2 * i], pf[2 * i + 1]}, bf16x2);
            pb[kp][2 * i] = pair[0];
            pb[kp][2 * i + 1] = pair[1];
            if constexpr (F32W) {
              const f32x2 rest = {pf[2 * i] - static_cast<float>(pair[0]), pf[2 * i + 1] - static_cast<float>(pair[1])};
              const bf16x2 lo = __builtin_convertvector(rest, bf16x2);
              pl[F32W ? kp : 0][2 * i] = lo[0];
              pl[F32W ? kp : 0][2 * i + 1] = lo[1];
            }
          }
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += pf[e];
          return sum;
        };
        // ---- O^T += V^T . P^T: k-step kp (16 tokens) outer, column block
        // inner, so an accumulator's MFMAs are several blocks apart.  V^T
        // fragments run VPF blocks ahead of their MFMAs.
        if constexpr (DSPLIT) {
          // This wave takes its d_c/4 columns of all four head groups: block
          // idx = (kp, cbl) is column block hg * CBW + cbl, whose swizzle
          // groups start hg * CBW / 2 groups in.  Accumulator slot j holds
          // head group (hg + j) mod 4, so slot 0 is the wave's own group,
          // whose P is already in registers: its MFMAs go first and run
          // while the waves meet at the barrier that publishes every P.
          // Every V^T fragment of the tile is read up front (the tile has
          // been visible since the ring barrier).
          const char* vbuf = buf + hg * (CBW / 2) * 128;
          constexpr int NV = 2 * CBW;
          bf16x8 va[NV];
#pragma unroll
          for (int idx = 0; idx < NV; ++idx) {
            const int kp = idx / CBW, cbl = idx % CBW;
            i16x4 t[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const char* a = vbuf + v_off[s][cbl & 1] + (cbl / 2) * 128 + kp * 16 * ROWB;
              t[s] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a));
            }
            __builtin_memcpy(&va[idx], &t[0], 8);
            __builtin_memcpy(reinterpret_cast<char*>(&va[idx]) + 8, &t[1], 8);
          }
          // P a k-step at a time: the exponentials of k-step 1 issue under the
          // own-group MFMAs of k-step 0
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            l_part += p_half(kp);
            ldsp[(kp * 2 + lh) * ROWS + hg * 32 + lr] = pb[kp];
            if constexpr (F32W) ldsp[4 * ROWS + (kp * 2 + lh) * ROWS + hg * 32 + lr] = pl[F32W ? kp : 0];
#pragma unroll
            for (int cbl = 0; cbl < CBW; ++cbl) {
              oacc[cbl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kp * CBW + cbl], pb[kp], oacc[cbl], 0, 0, 0);
              if constexpr (F32W)
                oacc[cbl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kp * CBW + cbl], pl[F32W ? kp : 0], oacc[cbl],
                                                                    0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          constexpr int NT2 = F32W ? 2 : 1;  // P terms
          bf16x8 px[NT2][2][4];
#pragma unroll
          for (int tm = 0; tm < NT2; ++tm)
#pragma unroll
            for (int kp = 0; kp < 2; ++kp)
#pragma unroll
              for (int j = 1; j < 4; ++j)
                px[tm][kp][j] = ldsp[tm * 4 * ROWS + (kp * 2 + lh) * ROWS + ((hg + j) & 3) * 32 + lr];
#pragma unroll
          for (int idx = 0; idx < NV; ++idx)
#pragma unroll
            for (int j = 1; j < 4; ++j)
#pragma unroll
              for (int tm = 0; tm < NT2; ++tm)
                oacc[j * CBW + idx % CBW] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[idx], px[tm][idx / CBW][j],
                                                                                   oacc[j * CBW + idx % CBW], 0, 0, 0);
        } else {
          l_part += p_half(0);
          l_part += p_half(1);
          constexpr int NV = 2 * CB;
          constexpr int VPF = 4;
          i16x4 vt[NV][2];
          auto load_v = [&](int idx) {
            const int kp = idx / CB, cb = idx % CB;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const char* a = buf + v_off[s][cb & 1] + (cb / 2) * 128 + kp * 16 * ROWB;
              vt[idx][s] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a));
            }
          };
#pragma unroll
          for (int idx = 0; idx < VPF; ++idx) load_v(idx);
#pragma unroll
          for (int idx = 0; idx < NV; ++idx) {
            if (idx + VPF < NV) load_v(idx + VPF);
            bf16x8 va;
            __builtin_memcpy(&va, &vt[idx][0], 8);
            __builtin_memcpy(reinterpret_cast<char*>(&va) + 8, &vt[idx][1], 8);
            oacc[idx % CB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[idx / CB], oacc[idx % CB], 0, 0, 0);
            if constexpr (F32W)
              oacc[idx % CB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pl[F32W ? idx / CB : 0], oacc[idx % CB], 0, 0, 0);
            // Keep source order: the reads of block idx + VPF stay above the MFMA
            // of block idx (the scheduler would otherwise sink them to their use).
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }();
    };
    for (int it = 0; it < ntile; it += 3) {
      tile(it, lds0, lds2);
      if (it + 1 < ntile) tile(it + 1, lds1, lds0);
      if (it + 2 < ntile) tile(it + 2, lds2, lds1);
    }
    if constexpr (MODE == 0) overflow = __ballot(!(l_part <= kOverflowMax)) != 0;
    return overflow;
  };

  const bool overflow = run_pass(std::integral_constant<int, 0>{});
  // workgroup OR of the waves' overflow flags, through the idle page buffer
  __syncthreads();
  if (lane == 0) reinterpret_cast<int*>(lds0)[wave] = overflow ? 1 : 0;
  __syncthreads();
  int any_overflow = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) any_overflow |= reinterpret_cast<const int*>(lds0)[w];
  if (any_overflow) {
    // Rare: some row's scores rose so far above its first visible key that
    // its sum of P passed kOverflowMax.  Redo the split exactly: true max
    // first, then accumulate.
    __syncthreads();
    m_run = -INFINITY;
    run_pass(std::integral_constant<int, 1>{});
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
    l_part = 0.f;
    run_pass(std::integral_constant<int, 2>{});
    __syncthreads();  // the epilogue stages through the tile buffers
  }

  // ---- combine the two token lanes of a head group (TW == 2)
  if constexpr (TW == 2) {
    __syncthreads();
    static_assert((HG * CB * 64 * 16 + HG * 64 * 2) * 4 <= TILE, "exchange must fit one page buffer");
    float* xo = reinterpret_cast<float*>(lds0);  // [hg][cb][lane][16]
    float* xs = xo + HG * CB * 64 * 16;          // [hg][lane][m, l]
    if (tw == 1) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<f32x4*>(&xo[((hg * CB + cb) * 64 + lane) * 16 + 4 * i]) =
              f32x4{oacc[cb][4 * i], oacc[cb][4 * i + 1], oacc[cb][4 * i + 2], oacc[cb][4 * i + 3]};
      xs[(hg * 64 + lane) * 2 + 0] = m_run;
      xs[(hg * 64 + lane) * 2 + 1] = l_part;
    }
    __syncthreads();
    if (tw == 1) return;
    const float m1 = xs[(hg * 64 + lane) * 2 + 0];
    const float l1 = xs[(hg * 64 + lane) * 2 + 1];
    const float m = fmaxf(m_run, m1);
    const float mu = m == -INFINITY ? 0.f : m;
    const float f0 = __builtin_amdgcn_exp2f(m_run - mu);
    const float f1 = __builtin_amdgcn_exp2f(m1 - mu);
    l_part = l_part * f0 + l1 * f1;
    m_run = m;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(&xo[((hg * CB + cb) * 64 + lane) * 16 + 4 * i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[cb][4 * i + e] = oacc[cb][4 * i + e] * f0 + o1[e] * f1;
      }
  }

  // ---- normalise and store, in float32: obar (or this split's partial slot)
  // row by row.  A lane holds four consecutive columns of one row per
  // (accumulator, group) and writes them as one 16-byte store.
  const float l = pair32_sum(l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (lrow < row_count && h2 == 0) {
    const float lse_v = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    const int64_t row_g = row_base + lrow;
    if (final_out) {
      if (p.lse != nullptr) p.lse[row_g] = lse_v;
    } else {
      p.ws_lse[static_cast<int64_t>(slot) * H + (row_g - static_cast<int64_t>(b) * H)] = lse_v;
    }
  }
  auto out_row = [&](int lr) -> int64_t {
    const int64_t row_g = row_base + lr;
    return final_out ? row_g : static_cast<int64_t>(slot) * H + (row_g - static_cast<int64_t>(b) * H);
  };
  float* const outf = final_out ? static_cast<float*>(p.out_latent) : p.ws_o;
  if constexpr (DSPLIT) {
    // This wave holds columns (hg * CBW + cbl) * 32 + 8g + 4h2 + e of rows
    // q * 32 + r32, q = (hg + j) mod 4, at oacc[j * CBW + cbl][4g + e]; every
    // row's 1/l goes through LDS (the P buffer is idle now).
    float* ldsl = reinterpret_cast<float*>(ldsp);
    if (h2 == 0) ldsl[lrow] = inv;
    __syncthreads();
    // float16 partials (decode at d_c = 512): this wave's 128 columns of a row
    // are one scaled quarter
    if constexpr (!PREFILL && CBW * 32 == 128) if (!final_out && p.half_partials) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int lr = ((hg + j) & 3) * 32 + r32;
        const float iv = ldsl[lr];
        float mx = 0.f;
#pragma unroll
        for (int cbl = 0; cbl < CBW; ++cbl)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, __builtin_fabsf(oacc[j * CBW + cbl][i]));
        mx = pair32_max(mx) * iv;
        int ex = 0;
        if (mx > 0.f && mx <= FLT_MAX) (void)frexpf(mx, &ex);
        const float sc = ldexpf(iv, -ex);  // 1/l and 2^-e in one (exact) factor
        if (lr < row_count) {
          const int64_t orow_i = out_row(lr);
          _Float16* hrow = reinterpret_cast<_Float16*>(p.ws_o) + orow_i * DC;
#pragma unroll
          for (int cbl = 0; cbl < CBW; ++cbl)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x16& o = oacc[j * CBW + cbl];
              const f16x2 lo = __builtin_convertvector((f32x2){o[4 * g4] * sc, o[4 * g4 + 1] * sc}, f16x2);
              const f16x2 hi = __builtin_convertvector((f32x2){o[4 * g4 + 2] * sc, o[4 * g4 + 3] * sc}, f16x2);
              uint2 pk;
              pk.x = __builtin_bit_cast(uint32_t, lo);
              pk.y = __builtin_bit_cast(uint32_t, hi);
              *reinterpret_cast<uint2*>(hrow + (hg * CBW + cbl) * 32 + 8 * g4 + 4 * h2) = pk;
            }
          if (h2 == 0) p.ws_exp[orow_i * (DC / 128) + hg] = ex;
        }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lr = ((hg + j) & 3) * 32 + r32;
      const float iv = ldsl[lr];
      if (lr < row_count) {
        float* orow = outf + out_row(lr) * DC;
#pragma unroll
        for (int cbl = 0; cbl < CBW; ++cbl)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x16& o = oacc[j * CBW + cbl];
            *reinterpret_cast<f32x4*>(orow + (hg * CBW + cbl) * 32 + 8 * g4 + 4 * h2) =
                f32x4{o[4 * g4] * iv, o[4 * g4 + 1] * iv, o[4 * g4 + 2] * iv, o[4 * g4 + 3] * iv};
          }
      }
    }
  } else {
    if (lrow < row_count) {
      float* orow = outf + out_row(lrow) * DC;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(orow + cb * 32 + 8 * g + 4 * h2) =
              f32x4{oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv, oacc[cb][4 * g + 2] * inv,
                    oacc[cb][4 * g + 3] * inv};
    }
  }
}

// K4: merge the splits of each sequence:  lse = log sum_s e^{lse_s},
// obar = sum_s e^{lse_s - lse} obar_s, in split order (deterministic).
// One workgroup per (sequence, 4 heads); 64 lanes per head.  Partials and
// obar are float32.
template <int DC, bool HALF>
__global__ void __launch_bounds__(256) merge_kernel(AttnParams p) {
  constexpr int PER = DC / 64;
  const int b = blockIdx.x;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int H = p.n_heads;
  const int L = p.split_pages;
  // prefix of split counts over sequences before b, and b's own count
  int base = 0, ns_b = 0;
  for (int b0 = 0; b0 <= b; b0 += 64) {
    const int bb = b0 + lane;
    int t = bb < p.batch ? p.seq_lens[bb] : 0;
    t = t < 0 ? 0 : t;
    const int pages = (t + kPage - 1) / kPage;
    const int ns = bb <= b ? pages / L + ((pages % L) != 0 ? 1 : 0) : 0;
    const int incl = wave_incl_scan(ns);
    if (b - b0 < 64) {
      ns_b = __shfl(ns, b - b0, 64);
      base += __shfl(incl, b - b0, 64) - ns_b;
    } else {
      base += __shfl(incl, 63, 64);
    }
  }
  if (head >= H || ns_b == 1 || base + ns_b > p.n_items) return;
  const int64_t row = static_cast<int64_t>(b) * H + head;
  float* out = static_cast<float*>(p.out_latent) + row * DC;
  const float* lse_s = p.ws_lse + static_cast<int64_t>(base) * H + head;  // split s at lse_s[s * H]
  const float* part = p.ws_o + (static_cast<int64_t>(base) * H + head) * DC + lane * PER;
  // float16 partials: element offsets as above, and the lane's quarter's exponent
  const _Float16* hpart = reinterpret_cast<const _Float16*>(p.ws_o) + (static_cast<int64_t>(base) * H + head) * DC +
                          lane * PER;
  const int32_t* pexp = HALF ? p.ws_exp + (static_cast<int64_t>(base) * H + head) * (DC / 128) + lane * PER / 128
                             : nullptr;
  // Splits go four a round, every load of a round issued before its use; the
  // first round's loads go out before the lse max, so they share its wait.
  constexpr int U = 4;
  float v[U][PER];
  float w[U];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a sequence with no splits (no tokens; then the workspace may be
      // empty) reads nothing
      if (s0 + u < ns_b) {
        if constexpr (HALF) {
          _Float16 hv[PER];
          __builtin_memcpy(hv, hpart + static_cast<int64_t>(s0 + u) * H * DC, PER * sizeof(_Float16));
          const int ex = pexp[static_cast<int64_t>(s0 + u) * H * (DC / 128)];
#pragma unroll
          for (int i = 0; i < PER; ++i) v[u][i] = ldexpf(static_cast<float>(hv[i]), ex);
        } else {
          __builtin_memcpy(v[u], part + static_cast<int64_t>(s0 + u) * H * DC, PER * sizeof(float));
        }
        w[u] = lse_s[static_cast<int64_t>(s0 + u) * H];
      } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) v[u][i] = 0;
        w[u] = -INFINITY;
      }
    }
  };
  load_round(0);
  // max of the splits' lse, the lanes taking splits side by side
  float m = -INFINITY;
  for (int s0 = 0; s0 < ns_b; s0 += 64)
    if (s0 + lane < ns_b) m = fmaxf(m, lse_s[static_cast<int64_t>(s0 + lane) * H]);
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s0 = 0; s0 < ns_b; s0 += U) {
      if (s0 > 0) load_round(s0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = __expf(w[u] - m);
        wsum += wu;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(wu, v[u][i], acc[i]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = acc[i] * inv;
  __builtin_memcpy(out + lane * PER, o, PER * sizeof(float));
  if (p.lse != nullptr && lane == 0) p.lse[row] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

template <int DC, int DR, int HG, int TW, bool PREFILL, bool F32W>
hipError_t launch_attn(const AttnParams& p, int64_t n_wg, hipStream_t s) {
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bf16_kernel<DC, DR, HG, TW, PREFILL, F32W>), dim3(static_cast<unsigned>(n_wg)),
                     dim3(64 * HG * TW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const AttnParams& p, hipStream_t s) {
  const int64_t n_wg = p.n_items * p.n_head_chunks;
  if (p.d_latent == 512 && p.d_rope == 64 && !p.f32w) return launch_attn<512, 64, 4, 1, false, false>(p, n_wg, s);
  if (p.d_latent == 256 && p.d_rope == 32) {
    if (p.f32w) return launch_attn<256, 32, 1, 2, false, true>(p, n_wg, s);
    return launch_attn<256, 32, 1, 2, false, false>(p, n_wg, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t s) {
  if (p.d_latent == 512 && p.d_rope == 64 && !p.f32w) return launch_attn<512, 64, 4, 1, true, false>(p, p.n_blocks, s);
  if (p.d_latent == 256 && p.d_rope == 32) {
    if (p.f32w) return launch_attn<256, 32, 4, 1, true, true>(p, p.n_blocks, s);
    return launch_attn<256, 32, 4, 1, true, false>(p, p.n_blocks, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const AttnParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  const dim3 grid(p.batch, (p.n_heads + 3) / 4);
  if (p.d_latent == 512 && p.half_partials)
    hipLaunchKernelGGL((merge_kernel<512, true>), grid, dim3(256), 0, s, p);
  else if (p.d_latent == 512)
    hipLaunchKernelGGL((merge_kernel<512, false>), grid, dim3(256), 0, s, p);
  else if (p.d_latent == 256 && !p.half_partials)
    hipLaunchKernelGGL((merge_kernel<256, false>), grid, dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mla
