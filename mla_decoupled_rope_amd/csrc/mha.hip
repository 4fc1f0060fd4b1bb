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
//   K^C[h][t][:] = W_UK[h] c_t,   V[h][t][:] = W_UV[h] c_t      (float16, head-major)
// one workgroup per (128 keys, head, K or V): D^T[i][t] = W[i][:] . c_t on
// v_mfma_f32_32x32x16_bf16, both operands staged through LDS in 64-wide
// slices of d_c, double buffered.
// Kernel 2 (mha_prefill_kernel): one workgroup per (sequence, head, 128
// queries); wave w owns queries 32w .. 32w+31.  Keys stream in 32-key tiles
// [K^C | R_t k^R_t | V] through a ring of three LDS buffers filled by
// buffer-load DMA (the position part straight from the cache rows); scores
// S^T = K . Q^T, online softmax in base 2 with O rescaled when a row's max
// rises, O^T += V^T . P^T with V^T from transpose reads.  Two workgroups
// share a CU (8 waves), so one wave's softmax overlaps another's MFMAs.
// The up-projected keys and values, the content part of q and P are float16
// (11-bit significands: this form rounds keys and values the absorbed form
// never forms, and float16 keeps that rounding 8x below bf16's); the position
// part stays bf16 from the cache and takes the bf16 MFMA into the same
// accumulator.  Keys and values must stay within float16 range (|x| < 65504).
#include <cfloat>

#include "common.hpp"

namespace mla {

namespace {

constexpr int kDh = 128;   // d_head = d_v of the materialised heads
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

struct SeqUnit {
  int b;
  int64_t u;         // unit index within the sequence
  int64_t key_base;  // first key row of the sequence in the workspace
  bool ok;
};

// Sequence b has n_q = cu_q[b+1] - cu_q[b] queries and T = q_start[b] + n_q
// keys.  Units per sequence: KIND 0 -> ceil(T / 128) key tiles, KIND 1 ->
// ceil(n_q / 128) * n_heads attention blocks.  Returns the sequence of a
// global unit index (sequence order) and its key offset sum_{b' < b} T_b'.
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
    const int64_t n = KIND == 0 ? (T + kBlk - 1) / kBlk : (nq + kBlk - 1) / kBlk * p.n_heads;
    const int64_t incl_u = wave_scan64(n), incl_k = wave_scan64(T);
    const int64_t lo = base_u + incl_u - n;
    const bool hit = n > 0 && unit >= lo && unit < lo + n;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __ffsll(static_cast<long long>(mask)) - 1;
      SeqUnit r;
      r.b = b0 + src;
      r.u = unit - __shfl(lo, src, 64);
      r.key_base = base_k + __shfl(incl_k, src, 64) - __shfl(T, src, 64);
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

// LDS slices are 128 rows x 64 bf16 (128-byte rows); 16-byte chunk ch of row
// r sits in slot ch ^ ((r >> 1) & 7), which puts the 16 rows of every
// fragment-read phase on distinct banks.
__device__ __forceinline__ int up_slot(int r, int ch) { return ch ^ ((r >> 1) & 7); }

template <int DC, int DR>
__global__ void __launch_bounds__(256) upproj_kernel(MhaParams p) {
  constexpr int KC = 64;            // d_c per slice
  constexpr int NSL = DC / KC;      // slices
  constexpr int RB = KC * 2;        // LDS row bytes
  constexpr int ROWB = (DC + DR) * 2;
  __shared__ __attribute__((aligned(16))) char lds_w[2][kDh * RB];
  __shared__ __attribute__((aligned(16))) char lds_c[2][kBlk * RB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SeqUnit su = find_unit<0>(p, blockIdx.x);
  if (!su.ok) return;
  const int b = __builtin_amdgcn_readfirstlane(su.b);
  const int t0 = __builtin_amdgcn_readfirstlane(static_cast<int>(su.u)) * kBlk;
  const int64_t key_base = su.key_base;
  const int nq = p.cu_q[b + 1] - p.cu_q[b];
  const int T = __builtin_amdgcn_readfirstlane(max(0, p.q_start[b]) + nq);
  const int tvalid = min(kBlk, T - t0);
  const int H = p.n_heads;
  const int yb = blockIdx.y;
  const bool is_v = yb >= H;
  const int h = is_v ? yb - H : yb;
  const bf16_t* w = static_cast<const bf16_t*>(is_v ? p.w_uv : p.w_uk) + static_cast<int64_t>(h) * kDh * DC;
  uint16_t* out = (is_v ? p.ws_v : p.ws_k) + (static_cast<int64_t>(h) * p.n_keys + key_base + t0) * kDh;

  // This thread's four 16-byte pieces of each slice: piece c = tid + 256 k is
  // row c / 8, chunk c % 8.  The cache row of a token row comes from the
  // block table (rows past the sequence repeat its last row).
  const char* cache = static_cast<const char*>(p.cache);
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const char* crow[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = (tid + 256 * k) >> 3;
    const int t = t0 + min(r, tvalid - 1);
    int page = bt[t / kPage];
    page = page < 0 || page >= p.num_pages ? 0 : page;
    crow[k] = cache + (static_cast<int64_t>(page) * kPage + t % kPage) * ROWB;
  }
  bf16x8 rw[4], rc[4];
  auto load = [&](int sl) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = tid + 256 * k;
      const int r = c >> 3, ch = c & 7;
      rw[k] = *reinterpret_cast<const bf16x8*>(w + static_cast<int64_t>(r) * DC + sl * KC + ch * 8);
      rc[k] = *reinterpret_cast<const bf16x8*>(crow[k] + (sl * KC + ch * 8) * 2);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = tid + 256 * k;
      const int r = c >> 3, ch = c & 7;
      *reinterpret_cast<bf16x8*>(&lds_w[buf][r * RB + up_slot(r, ch) * 16]) = rw[k];
      *reinterpret_cast<bf16x8*>(&lds_c[buf][r * RB + up_slot(r, ch) * 16]) = rc[k];
    }
  };
  // wave (wi, wt) takes output rows i = 64 wi .. +63 and tokens 64 wt .. +63
  const int wi = wave >> 1, wt = wave & 1;
  const int r32 = lane & 31, kh = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = f32x16{};
  load(0);
  store(0);
  __syncthreads();
  for (int sl = 0; sl < NSL; ++sl) {
    const int buf = sl & 1;
    if (sl + 1 < NSL) load(sl + 1);
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) {
      const int ch = ks * 2 + kh;
      bf16x8 fa[2], fc[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int r = wi * 64 + a * 32 + r32;
        fa[a] = *reinterpret_cast<const bf16x8*>(&lds_w[buf][r * RB + up_slot(r, ch) * 16]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = wt * 64 + c * 32 + r32;
        fc[c] = *reinterpret_cast<const bf16x8*>(&lds_c[buf][r * RB + up_slot(r, ch) * 16]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fc[c], acc[a][c], 0, 0, 0);
    }
    if (sl + 1 < NSL) store(buf ^ 1);
    __syncthreads();
  }
  // D[i][t]: lane (t = r32, half kh) holds i = 8g + 4kh + e at register 4g + e
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int t = wt * 64 + c * 32 + r32;
    if (t >= tvalid) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = wi * 64 + a * 32 + 8 * g + 4 * kh;
        uint2 pk;
        pk.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){acc[a][c][4 * g], acc[a][c][4 * g + 1]}, f16x2));
        pk.y = __builtin_bit_cast(uint32_t,
                                  __builtin_convertvector((f32x2){acc[a][c][4 * g + 2], acc[a][c][4 * g + 3]}, f16x2));
        *reinterpret_cast<uint2*>(out + static_cast<int64_t>(t) * kDh + i) = pk;
      }
  }
}

// -------------------------------------------------------------- attention

// LDS tile of 32 keys: K^C [32][128] (256-byte rows), the rotated position
// key [32][d_r], V [32][128].  Swizzles (16-byte chunk ch of row r):
//   K^C: slot ch ^ (r & 15)        -- 16 rows of a b128 read phase, distinct banks
//   k^R: slot ch ^ ((r >> 1) & 7)  (128-byte rows), ch ^ ((r >> 2) & 3) (64-byte rows)
//   V:   slot ch ^ 4 (r & 3)       -- the 4 rows of a transpose-read half-wave
__device__ __forceinline__ int kc_slot(int r, int ch) { return ch ^ (r & 15); }
template <int DR>
__device__ __forceinline__ int kr_slot(int r, int ch) {
  if constexpr (DR * 2 == 128) return ch ^ ((r >> 1) & 7);
  return ch ^ ((r >> 2) & 3);
}
__device__ __forceinline__ int v_slot(int r, int ch) { return ch ^ (4 * (r & 3)); }

template <int DC, int DR>
struct MhaTile {
  static constexpr int KC_B = kKeyTile * kDh * 2;  // 8 KB
  static constexpr int KR_B = kKeyTile * DR * 2;   // 4 KB (d_r 64) or 2 KB (d_r 32)
  static constexpr int V_B = kKeyTile * kDh * 2;   // 8 KB
  static constexpr int BYTES = KC_B + KR_B + V_B;
  static constexpr int KR_ROWS = 1024 / (DR * 2);  // key rows per 1 KiB DMA instruction
  static constexpr int N_KC = KC_B / 1024, N_KR = KR_B / 1024, N_V = V_B / 1024;
  static constexpr int N = N_KC + N_KR + N_V;      // wave instructions per tile
  static_assert(KR_B % 1024 == 0, "the position part must fill whole DMA instructions");
};

// The DMA of one key tile into an LDS buffer.  Instruction n of a tile:
// n < N_KC -> K^C rows 4n .. 4n+3; n < N_KC + N_V -> V rows; else the
// position part, KR_ROWS rows each.  Wave w issues instructions w, w + 4,
// w + 8, ...  Per-lane source offsets place each 16-byte chunk in its
// swizzled slot; rows past `valid` repeat the last valid row.
template <int DC, int DR>
__device__ __forceinline__ void mha_issue_tile(const MhaParams& p, int h, int64_t key_base, int t0, int valid, int page,
                                               char* dst, int wave, int lane) {
  using Tl = MhaTile<DC, DR>;
  constexpr int NW = 4;
  constexpr int NPW = (Tl::N + NW - 1) / NW;
  constexpr int ROWB = (DC + DR) * 2;
  const char* cache = static_cast<const char*>(p.cache);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_k + (static_cast<int64_t>(h) * p.n_keys + key_base + t0) * kDh, 0, Tl::KC_B, kBufWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_v + (static_cast<int64_t>(h) * p.n_keys + key_base + t0) * kDh, 0, Tl::V_B, kBufWord3);
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(cache) + (static_cast<int64_t>(page) * kPage + t0 % kPage) * ROWB + DC * 2, 0,
      kKeyTile * ROWB, kBufWord3);
  lds_char_t* ldst = reinterpret_cast<lds_char_t*>(reinterpret_cast<uintptr_t>(dst));
#pragma unroll
  for (int k = 0; k < NPW; ++k) {
    const int n = wave + NW * k;  // wave-uniform
    if (n >= Tl::N) break;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (n < Tl::N_KC) {
      const int r = 4 * n + (ln >> 4), slot = ln & 15;
      const int rs = min(r, valid - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, ldst + n * 1024, 16, rs * 256 + kc_slot(r, slot) * 16, 0, 0, 0);
    } else if (n < Tl::N_KC + Tl::N_V) {
      const int m = n - Tl::N_KC;
      const int r = 4 * m + (ln >> 4), slot = ln & 15;
      const int rs = min(r, valid - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, ldst + Tl::KC_B + Tl::KR_B + m * 1024, 16,
                                               rs * 256 + v_slot(r, slot) * 16, 0, 0, 0);
    } else {
      const int m = n - Tl::N_KC - Tl::N_V;
      constexpr int CPR = DR * 2 / 16;  // chunks per position row
      const int r = Tl::KR_ROWS * m + ln / CPR, slot = ln % CPR;
      const int rs = min(r, valid - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, ldst + Tl::KC_B + m * 1024, 16,
                                               rs * ROWB + kr_slot<DR>(r, slot) * 16, 0, 0, 0);
    }
  }
}

template <int DC, int DR>
__global__ void __launch_bounds__(256, 2) mha_prefill_kernel(MhaParams p) {
  using Tl = MhaTile<DC, DR>;
  constexpr int D = kDh + DR;      // score width
  constexpr int KS = D / 16;       // k-steps
  constexpr int KSC = kDh / 16;    // k-steps from K^C
  constexpr int ROWB = (DC + DR) * 2;
  constexpr int NW = 4;
  constexpr int NPW = (Tl::N + NW - 1) / NW;  // DMA instructions of the busiest wave
  __shared__ __attribute__((aligned(16))) char lds0[Tl::BYTES];
  __shared__ __attribute__((aligned(16))) char lds1[Tl::BYTES];
  __shared__ __attribute__((aligned(16))) char lds2[Tl::BYTES];

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
  const int h = u % H;
  const int qb = nqb - 1 - u / H;  // the latest query blocks (most keys) go first
  const int64_t key_base = su.key_base;
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
  // part converted to float16 (exact for bf16 values in float16 range)
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
        for (int e = 0; e < 8; ++e) y[e] = static_cast<_Float16>(static_cast<float>(x[e]));
        qc[ks < KSC ? ks : 0] = y;
      } else {
        qr[ks >= KSC ? ks - KSC : 0] = qvalid ? *reinterpret_cast<const bf16x8*>(ql + (d - kDh)) : bf16x8{};
      }
    }
  }

  // ---- tile DMA (mha_issue_tile)
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const int my_n = __builtin_amdgcn_readfirstlane((Tl::N - wave + NW - 1) / NW);  // this wave's count
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
    mha_issue_tile<DC, DR>(p, h, key_base, t0, min(kKeyTile, wg_last + 1 - t0), page, dst, wave, lane);
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
  static_assert(Tl::N >= NW * (NPW - 1), "every wave issues NPW or NPW - 1 instructions");

  // ---- per-lane LDS offsets (rows r32; K^C and k^R chunks ks*2 + h2)
  f32x16 oacc[kDh / 32];
#pragma unroll
  for (int c = 0; c < kDh / 32; ++c) oacc[c] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;

  if (ntile > 0) issue_tile(0, lds0);
  if (ntile > 1) issue_tile(1, lds1);
  auto tile = [&](int it, char* cur, char* nx2) {
    wait_tile(it + 1 < ntile);
    if (it + 2 < ntile) issue_tile(it + 2, nx2);
    const int t0 = it * kKeyTile;
    if (!wave_live || t0 > w_last) return;  // nothing this wave can see
    // ---- S^T = K . Q^T
    f32x16 sacc = f32x16{};
    constexpr int KPF = 4;
    bf16x8 ka[KS];
    auto load_k = [&](int ks) {
      const int ch = ks * 2 + h2;
      const char* a = ks < KSC ? cur + r32 * 256 + kc_slot(r32, ch) * 16
                               : cur + Tl::KC_B + r32 * (DR * 2) + kr_slot<DR>(r32, ch - 2 * KSC) * 16;
      ka[ks] = *reinterpret_cast<const bf16x8*>(a);
    };
#pragma unroll
    for (int ks = 0; ks < KPF; ++ks) load_k(ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + KPF < KS) load_k(ks + KPF);
      if (ks < KSC)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ka[ks]), qc[ks < KSC ? ks : 0], sacc,
                                                      0, 0, 0);
      else
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qr[ks >= KSC ? ks - KSC : 0], sacc, 0, 0, 0);
    }
    // ---- online softmax (base 2).  Lane (row r32, half h2) holds keys
    // t0 + 8g + 4h2 + e at register 4g + e.
    float sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
    if (t0 + kKeyTile - 1 > w_min) {  // the tile crosses some query's diagonal
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t0 + 8 * g + 4 * h2 + e > mpos) sv[4 * g + e] = -INFINITY;
    }
    float lmx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) lmx = fmaxf(lmx, sv[i]);
    const float m_new = fmaxf(m_run, pair32_max(lmx) * p.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = m_run == m_new ? 1.f : __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    if (alpha != 1.f) {
      l_part *= alpha;
#pragma unroll
      for (int c = 0; c < kDh / 32; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
    }
    f16x8 pb[2];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], p.scale_log2, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], p.scale_log2, -m_use));
      psum += p0 + p1;
      const f16x2 pair = __builtin_convertvector((f32x2){p0, p1}, f16x2);
      pb[i / 4][(2 * i) % 8] = pair[0];
      pb[i / 4][(2 * i) % 8 + 1] = pair[1];
    }
    l_part += psum;
    // ---- O^T += V^T . P^T.  Transpose read: supplier lane 16g + 4k + q reads
    // key row 16kp + 8s + 4(g/2) + k, columns cb*32 + 16(g%2) + 4q .. +3; lane
    // l receives column cb*32 + l%32 at keys 16kp + 8s + 4h + 0..3, the order
    // of its P registers 8kp + 4s + e.
    const char* vb = cur + Tl::KC_B + Tl::KR_B;
    const int vg = lane >> 4, vk = (lane >> 2) & 3, vq = lane & 3;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int cb = 0; cb < kDh / 32; ++cb) {
        i16x4 t[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int vrow = 16 * kp + 8 * s + 4 * (vg >> 1) + vk;
          const int ch = cb * 4 + 2 * (vg & 1) + (vq >> 1);
          const char* a = vb + vrow * 256 + v_slot(vrow, ch) * 16 + (vq & 1) * 8;
          t[s] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a));
        }
        f16x8 va;
        __builtin_memcpy(&va, &t[0], 8);
        __builtin_memcpy(reinterpret_cast<char*>(&va) + 8, &t[1], 8);
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[kp], oacc[cb], 0, 0, 0);
      }
  };
  for (int it = 0; it < ntile; it += 3) {
    tile(it, lds0, lds2);
    if (it + 1 < ntile) tile(it + 1, lds1, lds0);
    if (it + 2 < ntile) tile(it + 2, lds2, lds1);
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
  if (p.lse != nullptr && h2 == 0) p.lse[row] = l > 0.f ? (m_run + log2f(l)) * kLn2f : -INFINITY;
}

template <int DC, int DR>
hipError_t launch_mha(const MhaParams& p, hipStream_t s) {
  if (p.n_key_tiles > 0) {
    hipLaunchKernelGGL((upproj_kernel<DC, DR>), dim3(static_cast<unsigned>(p.n_key_tiles), 2 * p.n_heads), dim3(256),
                       0, s, p);
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
