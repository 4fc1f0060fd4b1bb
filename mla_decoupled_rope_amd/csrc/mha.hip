// Materialised-form causal prefill: up-project per-head keys and values from
// the latent cache, then run standard causal attention over them.
//
// "Multi-Head Latent Attention" (talalahmed.dev), the MLA dataflow: the per-
// head content key is W_UK c and the value is W_UV c, and each head's key is
// [content key ; shared rotated position key]; "AI decoupled RoPE MLA"
// (operatorworld.com), decoupled-RoPE section: the score is the sum of the
// content product and the rotated position product.  Both forms reach the
// same result ("ropeabsorb" README: absorption is exact); this one spends
//   2 n_h (d_h + d_r + d_v) flop per visible (query, key)
// plus 2 n_h (d_h + d_v) d_c flop per key for the up-projection, against
// 2 n_h (d_c + d_r + d_c) per pair in the absorbed form -- the cheaper form
// for a long causal chunk.
//
// Kernel 1 (upproj_kernel): for every key position t of every sequence,
//   K^C[h][t][:] = W_UK[h] c_t      (float16, [head][key][128])
//   V^T[h][:][t] = W_UV[h] c_t      (float16, [head][128][key], transposed)
// one workgroup per (256 keys, head) computes both: waves 0-1 the K^C rows,
// waves 2-3 the V^T rows, on v_mfma_f32_32x32x16_bf16, with the latent rows
// and both weight matrices staged through LDS in 32-wide slices of d_c (a
// ring of four, filled by buffer-load DMA).  Each sequence's keys take a
// range padded to a multiple of 128;
// the padding rows repeat the sequence's last latent, so every value in the
// workspace is finite.  V is stored transposed so that the P.V operand is a
// plain 16-byte LDS read (a transpose read would make the compiler wait for
// every LDS DMA in flight before it); within each 16-key group the keys are
// stored in the order 0-3, 8-11, 4-7, 12-15, the order in which a lane holds
// its softmax weights.
// Kernel 2 (mha_prefill_kernel): one workgroup per (sequence, head, 128
// queries); wave w owns queries 32w .. 32w+31.  Keys stream in 32-key tiles
// [K^C | R_t k^R_t | V^T] through a ring of four LDS buffers filled by
// buffer-load DMA (the position part straight from the cache rows); scores
// S^T = K . Q^T, online softmax in base 2 with O rescaled only when a row's
// max rises by more than 2^8, O^T += V^T . P^T.  Each wave issues the next
// tile's score MFMAs between the current tile's exponentials, and two
// workgroups share a CU (8 waves), so softmax work overlaps MFMAs.
// The up-projected keys and values, the content part of q and P are float16
// (11-bit significands: this form rounds keys and values the absorbed form
// never forms, and float16 keeps that rounding 8x below bf16's); the position
// part stays bf16 from the cache and takes the bf16 MFMA into the same
// accumulator.  Keys, values and the content query must stay within float16
// range: an element beyond it is stored as NaN, so the outputs it reaches are
// NaN rather than silently wrong.
#include <cfloat>

#include "common.hpp"

namespace mla {

namespace {

constexpr int kDh = 128;   // d_head = d_v of the materialised heads
constexpr int kUpPassHeads = 8;  // heads an XCD up-projects per pass over the keys
constexpr int kBlk = 128;  // keys per up-projection tile, queries per attention block
constexpr int kKeyTile = 32;
constexpr int kBufWord3 = 0x00020000;  // raw buffer resource, 32-bit format (gfx9 family)
constexpr float kLn2f = 0.69314718055994530942f;

constexpr int vmcnt_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ int64_t wave_scan64(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// A wave-uniform 64-bit value moved to scalar registers, so the buffer
// descriptors built from it stay scalar (a vector descriptor makes the
// compiler wrap every buffer load in a loop over the distinct values).
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(u)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(u >> 32)));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

struct SeqUnit {
  int b;
  int64_t u;         // unit index within the sequence
  int64_t key_base;  // first key row of the sequence in the workspace
  bool ok;
};

// Sequence b has n_q = cu_q[b+1] - cu_q[b] queries and T = q_start[b] + n_q
// keys, which occupy a workspace range of pad(T) = ceil(T / 128) * 128 keys.
// Units per sequence: KIND 0 -> ceil(T / 256) key tiles, KIND 1 ->
// ceil(n_q / 128) * n_heads attention blocks.  Returns the sequence of a
// global unit index (sequence order) and its key offset sum_{b' < b} pad(T_b').
template <int KIND>
__device__ SeqUnit find_unit(const MhaParams& p, int64_t unit) {
  const int lane = threadIdx.x & 63;
  int64_t base_u = 0, base_k = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int b = b0 + lane;
    int64_t nq = 0, T = 0;
    if (b < p.batch) {
      nq = max(0, p.cu_q[b + 1] - p.cu_q[b]);
      T = max(0, p.q_start[b]) + nq;
    }
    const int64_t n = KIND == 0 ? (T + 255) / 256 : (nq + kBlk - 1) / kBlk * p.n_heads;
    const int64_t Tp = (T + kBlk - 1) / kBlk * kBlk;
    const int64_t incl_u = wave_scan64(n), incl_k = wave_scan64(Tp);
    const int64_t lo = base_u + incl_u - n;
    const bool hit = n > 0 && unit >= lo && unit < lo + n;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __ffsll(static_cast<long long>(mask)) - 1;
      SeqUnit r;
      r.b = b0 + src;
      r.u = unit - __shfl(lo, src, 64);
      r.key_base = base_k + __shfl(incl_k, src, 64) - __shfl(Tp, src, 64);
      r.ok = true;
      return r;
    }
    base_u += __shfl(incl_u, 63, 64);
    base_k += __shfl(incl_k, 63, 64);
  }
  SeqUnit none{0, 0, 0, false};
  return none;
}

// ------------------------------------------------------------ up-projection

// One workgroup per (256 keys, head): 4 waves, wave (wt, wo) takes keys
// 128 wt .. +127 and wo = 0: the 128 K^C outputs (D[i][t] = W_UK[h][i] . c_t,
// W rows as the A operand), wo = 1: the 128 V outputs (D[t][i], c rows as the
// A operand, so a lane holds consecutive keys of one value dimension, the
// layout of V^T).  Each wave holds 4 x 4 blocks of 32 x 32 (AGPRs), so every
// fragment read from LDS serves four MFMAs.  d_c goes in 32-wide slices: a
// slice is the 256 latent rows and the 256 weight rows (W_UK[h] then
// W_UV[h]), 64 bytes each, 32 KiB, brought in by buffer-load DMA into a ring
// of four; chunk ch of row r sits in slot ch ^ ((r >> 2) & 3).
constexpr int kUpKeys = 256;  // keys per up-projection workgroup
constexpr int kUpSl = 32;     // d_c per slice

__device__ __forceinline__ int up_slot(int r, int ch) { return ch ^ ((r >> 2) & 3); }

// x where its float16 rounding is finite, NaN where it would overflow to
// infinity (|x| >= 65520, half way past 65504 rounds up): a key, value or
// content-query element outside the float16 range turns the outputs of its
// head that it reaches into NaN, never into finite wrong values (an infinite
// key could drop out of a softmax unnoticed).
__device__ __forceinline__ float f16_range(float x) { return __builtin_fabsf(x) < 65520.f ? x : __builtin_nanf(""); }

// D += A . B on an accumulator pinned to AGPRs (inline asm): the 256
// accumulator registers fill the AGPR file and the fragments the VGPRs; with
// the builtin the compiler splits the accumulators across both files and
// moves them every slice.
__device__ __forceinline__ void mfma_up(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <int DC, int DR>
__global__ void __launch_bounds__(256, 1) upproj_kernel(MhaParams p) {
  constexpr int NSL = DC / kUpSl;         // slices
  constexpr int RB = kUpSl * 2;           // LDS row bytes (64)
  constexpr int SLB = 2 * kUpKeys * RB;   // slice bytes: latent rows then weight rows
  constexpr int ROWB = (DC + DR) * 2;
  constexpr int NR = 4;                   // ring depth
  static_assert(NSL >= 2, "at least two slices");
  __shared__ __attribute__((aligned(16))) char lds_ring[NR * SLB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, kh = lane >> 5;
  // Placement: consecutive workgroups go to the 8 XCDs in turn; XCD x takes
  // heads x, x + 8, ... in passes of kUpPassHeads heads (their 2 MB of W_UK
  // and W_UV stay in the XCD's 4 MB L2 beside the latent tiles in flight; all
  // of its 16 heads' weights at once did not, and came back from memory for
  // every key tile).  A pass walks the key tiles with its heads innermost, so
  // a latent tile is read by consecutive workgroups, once per pass.
  const int H = p.n_heads;
  const int hpx = H / 8;
  int hpp = hpx < kUpPassHeads ? hpx : kUpPassHeads;  // heads per pass on one XCD: a divisor of hpx
  while (hpx % hpp != 0) --hpp;
  const int x = blockIdx.x;
  const int j8 = x >> 3;
  const int64_t per_pass = p.n_key_tiles * hpp;
  const int pass = static_cast<int>(j8 / per_pass);
  const int64_t rem = j8 % per_pass;
  const int h = (pass * hpp + static_cast<int>(rem % hpp)) * 8 + (x & 7);
  const SeqUnit su = find_unit<0>(p, rem / hpp);
  if (!su.ok) return;
  const int b = __builtin_amdgcn_readfirstlane(su.b);
  const int t0 = __builtin_amdgcn_readfirstlane(static_cast<int>(su.u)) * kUpKeys;
  const int64_t key_base = uniform_i64(su.key_base);
  const int nq = p.cu_q[b + 1] - p.cu_q[b];
  const int T = __builtin_amdgcn_readfirstlane(max(0, p.q_start[b]) + nq);
  const int Tp = (T + kBlk - 1) / kBlk * kBlk - t0;  // rows of this tile inside the padded range

  // ---- DMA.  Instruction n of a slice: n < 16 -> latent rows 16n .. 16n+15
  // (one cache page: 16 consecutive keys, rows past the sequence repeat its
  // last row); n >= 16 -> weight rows 16(n-16) .. +15.  Wave w issues n = w +
  // 4k, k = 0..7: latent for k < 4, W_UK for k = 4, 5, W_UV for k = 6, 7.  Each
  // lane's source offset within the instruction's buffer is fixed; slices
  // advance through the scalar offset.
  const char* cache = static_cast<const char*>(p.cache);
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  __amdgpu_buffer_rsrc_t rc[4];
  uint32_t off[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = wave + 4 * k;
    const int row = 16 * n + (lane >> 2), slot = lane & 3;
    const int ts = min(t0 + row, T - 1);
    const int first = min(t0 + 16 * n, T - 1);  // every row of the instruction is in this row's page
    int page = bt[first / kPage];
    page = page < 0 || page >= p.num_pages ? 0 : page;
    page = __builtin_amdgcn_readfirstlane(page);
    rc[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(cache) + static_cast<int64_t>(page) * kPage * ROWB, 0,
                                              kPage * ROWB, kBufWord3);
    off[k] = static_cast<uint32_t>((ts % kPage) * ROWB + up_slot(row, slot) * 16);
  }
  const __amdgpu_buffer_rsrc_t rwk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(static_cast<const bf16_t*>(p.w_uk)) + static_cast<int64_t>(h) * kDh * DC, 0, kDh * DC * 2,
      kBufWord3);
  const __amdgpu_buffer_rsrc_t rwv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(static_cast<const bf16_t*>(p.w_uv)) + static_cast<int64_t>(h) * kDh * DC, 0, kDh * DC * 2,
      kBufWord3);
#pragma unroll
  for (int k = 4; k < 8; ++k) {
    const int n = wave + 4 * k - 16;
    const int row = 16 * n + (lane >> 2), slot = lane & 3;
    off[k] = static_cast<uint32_t>((row % kDh) * DC * 2 + up_slot(row, slot) * 16);
  }
  auto buf = [&](int s) { return lds_ring + (s % NR) * SLB; };
  auto issue = [&](int s) {
    lds_char_t* dst = reinterpret_cast<lds_char_t*>(reinterpret_cast<uintptr_t>(buf(s)));
    const int so = s * RB;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int n = wave + 4 * k;
      const __amdgpu_buffer_rsrc_t r = k < 4 ? rc[k] : (k < 6 ? rwk : rwv);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + n * 1024, 16, off[k], so, 0, 0);
    }
  };

  // ---- fragments: wave (wt, wo); A rows and B rows of block a / c are
  // base + 32 a + r32; chunk 2 ks + kh
  const int wt = wave & 1, wo = wave >> 1;
  const int a_base = wo == 0 ? kUpKeys * RB : wt * 128 * RB;                 // W_UK rows, or latent rows
  const int b_base = wo == 0 ? wt * 128 * RB : (kUpKeys + 128) * RB;        // latent rows, or W_UV rows
  int foff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) foff[ks] = r32 * RB + up_slot(r32, 2 * ks + kh) * 16;
  // Only LDS reads (ordered by s_waitcnt) write the fragment registers: the
  // inline-asm MFMAs are invisible to the hazard recognizer, so a VALU write
  // (a register copy, say) feeding one could be read stale.
  bf16x8 fa[2][4], fb[2][4];
  auto load_frags = [&](const char* sl) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        fa[ks][a] = *reinterpret_cast<const bf16x8*>(sl + a_base + foff[ks] + a * 32 * RB);
        fb[ks][a] = *reinterpret_cast<const bf16x8*>(sl + b_base + foff[ks] + a * 32 * RB);
      }
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x16{};

  // ---- slices: step s waits for slice s+1 and meets the barrier (after which
  // buffer (s+3) % 4 = (s-1) % 4 is free), issues slice s+3 (this wave's turn
  // after its a-row `wave` of MFMAs), computes slice s from the fragments
  // read at the end of step s-1, and reads slice s+1's fragments.
  issue(0);
  issue(1);
  if (NSL > 2) issue(2);
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(NSL > 2 ? 16 : 8));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  load_frags(buf(0));
  for (int s = 0; s < NSL; ++s) {
    if (s + 1 < NSL) {
      // this wave's DMAs of slice s+2 may stay in flight
      if (s + 2 < NSL) __builtin_amdgcn_s_waitcnt(vmcnt_wait(8));
      else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      asm volatile("s_barrier" ::: "memory");
    }
    const bool dma = s + 3 < NSL;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int c = 0; c < 4; ++c) mfma_up(acc[a][c], fa[ks][a], fb[ks][c]);
        if (ks == 0 && a == wave && dma) issue(s + 3);
      }
    if (s + 1 < NSL) load_frags(buf(s + 1));
  }

  // ---- store, rows of the padded range only.  The tile goes through the idle
  // ring first (K^C as its 256-byte rows [t][i], V^T as 512-byte rows [i][t] in
  // the stored key order), so the global writes are whole rows: the K^C tile
  // is one contiguous 64 KiB run, each V^T row 512 contiguous bytes.
  auto h2pack = [](float u, float v) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f16_range(u), f16_range(v)}, f16x2));
  };
  constexpr int KROW = kDh * 2;        // K^C row bytes (256)
  constexpr int VROW = kUpKeys * 2;    // V^T row bytes in the tile (512)
  char* stk = lds_ring;                // K^C tile, 64 KiB
  char* stv = lds_ring + kUpKeys * KROW;  // V^T tile, 64 KiB
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave is done with the ring
  if (wo == 0) {
    // D[i][t]: lane (t = r32, half kh) holds i = 32a + 8g + 4kh + e at register 4g + e.
    // 8-byte pieces of row t; the piece index is XOR-swizzled by the row so the
    // 32 rows of a store land on distinct banks.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = wt * 128 + c * 32 + r32;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 pk;
          pk.x = h2pack(acc[a][c][4 * g], acc[a][c][4 * g + 1]);
          pk.y = h2pack(acc[a][c][4 * g + 2], acc[a][c][4 * g + 3]);
          const int piece = (a * 32 + 8 * g + 4 * kh) / 4;  // 0..31
          *reinterpret_cast<uint2*>(stk + t * KROW + ((piece ^ (t & 31)) * 8)) = pk;
        }
    }
  } else {
    // D[t][i]: lane (i = r32, half kh) holds t = 32a + 16q + 8s + 4kh + e at
    // register 4(2q + s) + e; it goes to position 16q + 8kh + 4s + e of its
    // 16-key group, a 16-byte piece of row i (XOR-swizzled by the row).
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x16& v = acc[a][c];
          uint4 pk;
          pk.x = h2pack(v[8 * q], v[8 * q + 1]);
          pk.y = h2pack(v[8 * q + 2], v[8 * q + 3]);
          pk.z = h2pack(v[8 * q + 4], v[8 * q + 5]);
          pk.w = h2pack(v[8 * q + 6], v[8 * q + 7]);
          const int i = c * 32 + r32;
          const int piece = (wt * 128 + a * 32 + 16 * q + 8 * kh) / 8;  // 0..31
          *reinterpret_cast<uint4*>(stv + i * VROW + ((piece ^ (i & 31)) * 16)) = pk;
        }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // K^C: rows t < Tp, 16 pieces of 16 bytes a row, 256 threads -> 16 rows a pass
  {
    char* out = reinterpret_cast<char*>(p.ws_k + (static_cast<int64_t>(h) * p.n_keys + key_base + t0) * kDh);
    const int rows = min(kUpKeys, Tp);
#pragma unroll 4
    for (int r0 = 0; r0 < kUpKeys; r0 += 16) {
      const int t = r0 + (tid >> 4), q16 = tid & 15;
      if (t < rows) {
        // 16-byte piece q16 = 8-byte pieces 2 q16, 2 q16 + 1 (swizzled separately)
        const uint2 lo = *reinterpret_cast<const uint2*>(stk + t * KROW + (((2 * q16) ^ (t & 31)) * 8));
        const uint2 hi = *reinterpret_cast<const uint2*>(stk + t * KROW + (((2 * q16 + 1) ^ (t & 31)) * 8));
        *reinterpret_cast<uint4*>(out + static_cast<int64_t>(t) * KROW + q16 * 16) = uint4{lo.x, lo.y, hi.x, hi.y};
      }
    }
  }
  // V^T: 128 rows, the first min(256, Tp) keys of each (Tp is a multiple of 128)
  {
    uint16_t* out = p.ws_v + static_cast<int64_t>(h) * kDh * p.n_keys + key_base + t0;
    const int pieces = min(kUpKeys, Tp) / 8;  // 16-byte pieces a row: 16 or 32
#pragma unroll 4
    for (int r0 = 0; r0 < kDh; r0 += 8) {
      const int i = r0 + (tid >> 5), pc = tid & 31;
      if (pc < pieces)
        *reinterpret_cast<uint4*>(out + static_cast<int64_t>(i) * p.n_keys + pc * 8) =
            *reinterpret_cast<const uint4*>(stv + i * VROW + ((pc ^ (i & 31)) * 16));
    }
  }
}

// -------------------------------------------------------------- attention

// LDS tile of 32 keys: K^C [32][128] (256-byte rows), the rotated position
// key [32][d_r], V^T [128][32] (64-byte rows).  Swizzles (16-byte chunk ch of
// row r), each putting the 16 rows of a b128 read phase on distinct banks:
//   K^C: slot ch ^ (r & 15)
//   k^R: slot ch ^ ((r >> 1) & 7)  (128-byte rows), ch ^ ((r >> 2) & 3) (64-byte rows)
//   V^T: slot ch ^ ((r >> 2) & 3)
__device__ __forceinline__ int kc_slot(int r, int ch) { return ch ^ (r & 15); }
template <int DR>
__device__ __forceinline__ int kr_slot(int r, int ch) {
  if constexpr (DR * 2 == 128) return ch ^ ((r >> 1) & 7);
  return ch ^ ((r >> 2) & 3);
}
__device__ __forceinline__ int vt_slot(int r, int ch) { return ch ^ ((r >> 2) & 3); }

template <int DC, int DR>
struct MhaTile {
  static constexpr int KC_B = kKeyTile * kDh * 2;  // 8 KB
  static constexpr int KR_B = kKeyTile * DR * 2;   // 4 KB (d_r 64) or 2 KB (d_r 32)
  static constexpr int V_B = kKeyTile * kDh * 2;   // 8 KB
  static constexpr int BYTES = KC_B + KR_B + V_B;
  static constexpr int KR_ROWS = 1024 / (DR * 2);  // key rows per 1 KiB DMA instruction
  static constexpr int N_KC = KC_B / 1024, N_KR = KR_B / 1024, N_V = V_B / 1024;
  static constexpr int N = N_KC + N_KR + N_V;      // wave instructions per tile
  static constexpr int NW = 4;
  static constexpr int NPW = (N + NW - 1) / NW;    // instructions of the busiest wave
  static_assert(KR_B % 1024 == 0, "the position part must fill whole DMA instructions");
  static_assert(N >= NW * (NPW - 1), "every wave issues NPW or NPW - 1 instructions");
};

// The DMA of one key tile into an LDS buffer.  Instruction n of a tile:
// n < N_KC -> K^C rows 4n .. 4n+3; n < N_KC + N_V -> V^T rows (value
// dimensions) 16m .. 16m+15; else the position part, KR_ROWS key rows each.
// Wave w issues instructions w, w + 4, w + 8, ...  Every tile lies inside
// its sequence's padded key range and inside one cache page, so a lane's
// source offset within an instruction's buffer depends only on the lane,
// the instruction and the workspace row length: it is computed once.
template <int DC, int DR>
__device__ __forceinline__ uint32_t mha_dma_offset(int n, int lane, int64_t n_keys) {
  using Tl = MhaTile<DC, DR>;
  constexpr int ROWB = (DC + DR) * 2;
  if (n < Tl::N_KC) {
    const int r = 4 * n + (lane >> 4), slot = lane & 15;
    return static_cast<uint32_t>(r * 256 + kc_slot(r, slot) * 16);
  }
  if (n < Tl::N_KC + Tl::N_V) {
    const int m = n - Tl::N_KC;
    const int r = 16 * m + (lane >> 2), slot = lane & 3;
    return static_cast<uint32_t>(r * n_keys * 2 + vt_slot(r, slot) * 16);
  }
  const int m = n - Tl::N_KC - Tl::N_V;
  constexpr int CPR = DR * 2 / 16;  // chunks per position row
  const int r = Tl::KR_ROWS * m + lane / CPR, slot = lane % CPR;
  return static_cast<uint32_t>(r * ROWB + kr_slot<DR>(r, slot) * 16);
}

// rk / rv cover the sequence's K^C rows / V^T columns of head h; the tile
// starts t0 keys in (scalar offsets t0 * 256 and t0 * 2 bytes).
template <int DC, int DR>
__device__ __forceinline__ void mha_issue_tile(const MhaParams& p, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                               int t0, int page, char* dst, int wave,
                                               const uint32_t (&off)[MhaTile<DC, DR>::NPW]) {
  using Tl = MhaTile<DC, DR>;
  constexpr int ROWB = (DC + DR) * 2;
  const char* cache = static_cast<const char*>(p.cache);
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(cache) + (static_cast<int64_t>(page) * kPage + t0 % kPage) * ROWB + DC * 2, 0,
      kKeyTile * ROWB, kBufWord3);
  lds_char_t* ldst = reinterpret_cast<lds_char_t*>(reinterpret_cast<uintptr_t>(dst));
#pragma unroll
  for (int k = 0; k < Tl::NPW; ++k) {
    const int n = wave + Tl::NW * k;  // wave-uniform
    if (n >= Tl::N) break;
    if (n < Tl::N_KC) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, ldst + n * 1024, 16, off[k], t0 * (kDh * 2), 0, 0);
    } else if (n < Tl::N_KC + Tl::N_V) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, ldst + Tl::KC_B + Tl::KR_B + (n - Tl::N_KC) * 1024, 16, off[k],
                                               t0 * 2, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, ldst + Tl::KC_B + (n - Tl::N_KC - Tl::N_V) * 1024, 16, off[k], 0,
                                               0, 0);
    }
  }
}

template <int DC, int DR>
__global__ void __launch_bounds__(256, 2) mha_prefill_kernel(MhaParams p) {
  using Tl = MhaTile<DC, DR>;
  constexpr int D = kDh + DR;      // score width
  constexpr int KS = D / 16;       // k-steps
  constexpr int KSC = kDh / 16;    // k-steps from K^C
  constexpr int NW = Tl::NW;
  constexpr int NPW = Tl::NPW;
  __shared__ __attribute__((aligned(16))) char lds_ring[4 * Tl::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h2 = lane >> 5;
  const int H = p.n_heads;

  const SeqUnit su = find_unit<1>(p, blockIdx.x);
  if (!su.ok) return;
  const int b = __builtin_amdgcn_readfirstlane(su.b);
  const int nq = __builtin_amdgcn_readfirstlane(p.cu_q[b + 1] - p.cu_q[b]);
  const int q_first = __builtin_amdgcn_readfirstlane(p.cu_q[b]);
  const int qpos0 = __builtin_amdgcn_readfirstlane(max(0, p.q_start[b]));
  const int nqb = (nq + kBlk - 1) / kBlk;
  const int u = __builtin_amdgcn_readfirstlane(static_cast<int>(su.u));
  // Placement: a sequence's nqb * H units start at a multiple of 8 (H is), and
  // consecutive workgroups go to the 8 XCDs in turn, so unit u runs on XCD
  // u % 8.  Each XCD takes the query blocks of heads u % 8, u % 8 + 8, ... one
  // head at a time, so the blocks that stream the same keys and values run
  // together and share that XCD's L2.  Within a head the latest query blocks
  // (most keys) go first.
  const int j8 = u >> 3;
  const int h = (j8 / nqb) * 8 + (u & 7);
  const int qb = nqb - 1 - j8 % nqb;
  const int64_t key_base = uniform_i64(su.key_base);
  // this lane's query (row r32 of the wave), its position, validity
  const int jq = qb * kBlk + wave * 32 + r32;
  const bool qvalid = jq < nq;
  const int mpos = qpos0 + jq;
  // wave-uniform extent: the last key any query of the workgroup / of this wave sees
  const int wg_last = qpos0 + min(nq, (qb + 1) * kBlk) - 1;
  const int w_first_q = qb * kBlk + wave * 32;
  const bool wave_live = w_first_q < nq;
  const int w_last = qpos0 + min(nq, w_first_q + 32) - 1;
  const int w_min = qpos0 + w_first_q;  // position of the wave's first query
  const int ntile = (wg_last + kKeyTile) / kKeyTile;

  // ---- Q fragments (B operand): row r32, d = ks*16 + 8*h2 .. +7; the content
  // part converted to float16 (exact for bf16 values of magnitude 2^-17 ..
  // 65504; NaN beyond float16 range)
  f16x8 qc[KSC];
  bf16x8 qr[KS - KSC];
  {
    const bf16_t* qn = static_cast<const bf16_t*>(p.q_nope) + (static_cast<int64_t>(q_first + jq) * H + h) * kDh;
    const bf16_t* ql = static_cast<const bf16_t*>(p.q_lat) + (static_cast<int64_t>(q_first + jq) * H + h) * (DC + DR) + DC;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d = ks * 16 + 8 * h2;
      if (ks < KSC) {
        const bf16x8 x = qvalid ? *reinterpret_cast<const bf16x8*>(qn + d) : bf16x8{};
        f16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = static_cast<_Float16>(f16_range(static_cast<float>(x[e])));
        qc[ks < KSC ? ks : 0] = y;
      } else {
        qr[ks >= KSC ? ks - KSC : 0] = qvalid ? *reinterpret_cast<const bf16x8*>(ql + (d - kDh)) : bf16x8{};
      }
    }
  }

  // ---- tile DMA
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const int my_n = __builtin_amdgcn_readfirstlane((Tl::N - wave + NW - 1) / NW);  // this wave's count
  uint32_t doff[NPW];
#pragma unroll
  for (int k = 0; k < NPW; ++k) doff[k] = mha_dma_offset<DC, DR>(min(wave + NW * k, Tl::N - 1), lane, p.n_keys);
  const int Tpad = (wg_last + kBlk) / kBlk * kBlk;  // keys of the padded range this workgroup may read
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_k + (static_cast<int64_t>(h) * p.n_keys + key_base) * kDh, 0,
      static_cast<int>(static_cast<uint32_t>(min(static_cast<int64_t>(Tpad) * kDh * 2, int64_t{0xffffffff}))), kBufWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_v + static_cast<int64_t>(h) * kDh * p.n_keys + key_base, 0,
      static_cast<int>(static_cast<uint32_t>(((kDh - 1) * p.n_keys + Tpad) * 2)), kBufWord3);
  // Page ids 64 at a time: lane j holds page (ids_base + j); a tile reads its
  // id with readlane, so the tile loop issues no other vector loads (a load
  // there would make the compiler wait for every DMA in flight).
  int ids_base = 0;
  auto load_ids = [&](int first) {
    const int pg = first + lane;
    const int id = pg < p.max_pages ? bt[pg] : 0;
    return id < 0 || id >= p.num_pages ? 0 : id;
  };
  int ids = load_ids(0);
  auto issue_tile = [&](int it, char* dst) {
    const int t0 = it * kKeyTile;
    const int pg = t0 / kPage;
    if (pg - ids_base >= 64) {
      ids_base = pg;
      ids = load_ids(pg);
    }
    const int page = __builtin_amdgcn_readlane(ids, pg - ids_base);
    mha_issue_tile<DC, DR>(p, rk, rv, t0, page, dst, wave, doff);
  };
  auto wait_tile = [&](bool newer_in_flight) {
    // this wave's instructions of the newer tile may stay in flight
    if (newer_in_flight) {
      if (my_n == NPW) __builtin_amdgcn_s_waitcnt(vmcnt_wait(NPW));
      else __builtin_amdgcn_s_waitcnt(vmcnt_wait(NPW - 1));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // ---- per-lane LDS read offsets: K^C / k^R row r32, chunk 2 ks + h2; V^T
  // row 32 cb + r32, chunk 2 kp + h2
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int ch = ks * 2 + h2;
    koff[ks] = ks < KSC ? r32 * 256 + kc_slot(r32, ch) * 16
                        : Tl::KC_B + r32 * (DR * 2) + kr_slot<DR>(r32, ch - 2 * KSC) * 16;
  }
  int voff[2];
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) voff[kp] = Tl::KC_B + Tl::KR_B + r32 * 64 + vt_slot(r32, 2 * kp + h2) * 16;

  f32x16 oacc[kDh / 32];
#pragma unroll
  for (int c = 0; c < kDh / 32; ++c) oacc[c] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;

  // ---- the pipeline.  Tiles go round a ring of four LDS buffers.  Step it
  // waits for tile it+1, meets the other waves at the barrier (after which
  // nobody reads buffer (it+3) % 4 = (it-1) % 4 any more) and issues tile
  // it+3 there; then it issues the score MFMAs of tile it+1 with the
  // exponentials of tile it between them, and ends with tile it's P.V.
  // The waves see a prefix of the tiles: wave_tiles of them.
  const int wave_tiles = wave_live ? w_last / kKeyTile + 1 : 0;
  auto buf = [&](int it) { return lds_ring + (it & 3) * Tl::BYTES; };
  auto qk_load = [&](const char* cur, bf16x8 (&ka)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(cur + koff[ks]);
  };
  auto qk_step = [&](int ks, const bf16x8 (&ka)[KS], f32x16 s) {
    if (ks < KSC)
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ka[ks]), qc[ks < KSC ? ks : 0], s, 0, 0,
                                                    0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qr[ks >= KSC ? ks - KSC : 0], s, 0, 0, 0);
  };

  for (int k = 0; k < 3 && k < ntile; ++k) issue_tile(k, buf(k));
  {
    // tile 0 lands; tiles 1 and 2 may stay in flight
    const int newer = min(2, ntile - 1);
    const int n = newer * my_n;
    if (n >= 2 * NPW) __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * NPW));
    else if (n >= 2 * NPW - 2) __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * NPW - 2));
    else if (n >= NPW) __builtin_amdgcn_s_waitcnt(vmcnt_wait(NPW));
    else if (n >= NPW - 1) __builtin_amdgcn_s_waitcnt(vmcnt_wait(NPW - 1));
    else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  f32x16 sacc = f32x16{};
  if (wave_tiles > 0) {
    bf16x8 ka[KS];
    qk_load(buf(0), ka);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc = qk_step(ks, ka, sacc);
  }

  for (int it = 0; it < ntile; ++it) {
    if (it + 1 < ntile) {
      wait_tile(it + 2 < ntile);
      if (it + 3 < ntile) issue_tile(it + 3, buf(it + 3));
    }
    if (it >= wave_tiles) continue;  // keeps meeting the barriers
    const int t0 = it * kKeyTile;
    const char* cur = buf(it);
    // V^T fragments of tile it, read first: they have the whole step to land
    f16x8 va[2][kDh / 32];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int cb = 0; cb < kDh / 32; ++cb)
        va[kp][cb] = *reinterpret_cast<const f16x8*>(cur + voff[kp] + cb * 32 * 64);
    __builtin_amdgcn_sched_barrier(0);
    // ---- row max of tile it.  Lane (row r32, half h2) holds keys
    // t0 + 8g + 4h2 + e at register 4g + e.
    float sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
    if (t0 + kKeyTile - 1 > w_min) {  // the tile crosses some query's diagonal (or the sequence end)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t0 + 8 * g + 4 * h2 + e > mpos) sv[4 * g + e] = -INFINITY;
    }
    // The row's reference m_run moves only when this tile's max exceeds it by
    // more than 8 (base 2): weights up to 2^8 stay far inside float16 and the
    // float32 sums, and O is rescaled on few tiles instead of on every rise.
    float lmx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) lmx = fmaxf(lmx, sv[i]);
    const float m_tile = pair32_max(lmx) * p.scale_log2;
    if (m_tile > m_run + 8.f) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_tile);  // 0 while m_run is -inf
      m_run = m_tile;
      l_part *= alpha;
#pragma unroll
      for (int c = 0; c < kDh / 32; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    // ---- scores of tile it+1 (MFMA) with the weights of tile it (VALU)
    // between them: k-step ks carries key pair ks of this lane.
    const bool next = it + 1 < wave_tiles;
    f16x8 pb[2];
    float psum = 0.f;
    auto weights = [&](int i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], p.scale_log2, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], p.scale_log2, -m_use));
      psum += p0 + p1;
      const f16x2 pair = __builtin_convertvector((f32x2){p0, p1}, f16x2);
      pb[i / 4][(2 * i) % 8] = pair[0];
      pb[i / 4][(2 * i) % 8 + 1] = pair[1];
    };
    if (next) {
      bf16x8 ka[KS];
      qk_load(buf(it + 1), ka);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sn = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sn = qk_step(ks, ka, sn);
        if (ks < 8) weights(ks);
      }
#pragma unroll
      for (int i = KS; i < 8; ++i) weights(i);
      sacc = sn;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) weights(i);
    }
    l_part += psum;
    // ---- O^T += V^T . P^T.  In k-step kp, position 8h + 4s + e of the
    // sixteen holds key 16kp + 8s + 4h + e on both sides: the V^T rows store
    // their keys in that order, and pb[kp] packs this lane's registers
    // 4(2kp + s) + e.
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int cb = 0; cb < kDh / 32; ++cb)
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[kp][cb], pb[kp], oacc[cb], 0, 0, 0);
  }
  // ---- normalise and store o (float32) and lse
  const float l = pair32_sum(l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (!qvalid) return;
  const int64_t row = static_cast<int64_t>(q_first + jq) * H + h;
  float* o = p.out + row * kDh;
#pragma unroll
  for (int cb = 0; cb < kDh / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v{oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv, oacc[cb][4 * g + 2] * inv,
                    oacc[cb][4 * g + 3] * inv};
      *reinterpret_cast<f32x4*>(o + cb * 32 + 8 * g + 4 * h2) = v;
    }
  // (no visible key: -inf; a NaN sum -- an input out of float16 range -- stays NaN)
  if (p.lse != nullptr && h2 == 0) p.lse[row] = l == 0.f ? -INFINITY : (m_run + log2f(l)) * kLn2f;
}

template <int DC, int DR>
hipError_t launch_mha(const MhaParams& p, hipStream_t s) {
  if (p.n_key_tiles > 0) {
    hipLaunchKernelGGL((upproj_kernel<DC, DR>), dim3(static_cast<unsigned>(p.n_key_tiles * p.n_heads)), dim3(256), 0,
                       s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.n_q_blocks > 0)
    hipLaunchKernelGGL((mha_prefill_kernel<DC, DR>), dim3(static_cast<unsigned>(p.n_q_blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mha_prefill(const MhaParams& p, hipStream_t s) {
  if (p.d_latent == 512 && p.d_rope == 64) return launch_mha<512, 64>(p, s);
  if (p.d_latent == 256 && p.d_rope == 32) return launch_mha<256, 32>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
