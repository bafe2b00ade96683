// Mixed-batch attention over a paged, block-quantized KV cache, for gfx950.
//
// Operations follow the MBufo page "自研RDNA高併發推論引擎 以AI Max+ 395為範例":
//   section 1  -- chunk rows and decode rows share one ForwardBatch and one
//                 attention kernel (one launch serves both row kinds here);
//   section 2  -- KV modes table: 32-value blocks with one fp16 scale, 34 bytes
//                 (8-bit codes) or 18 bytes (4-bit codes), bit-exact codec; the
//                 table's fp16 row is the unquantized 64-byte format.
//
// Kernels:
//   append_kernel           -- encode new K/V rows into blocks at their page slots.
//   mixed_attention_kernel  -- one launch over a flat list of work items: chunk
//                              tiles first (heavy), then the decode stream.
//   decode_attention_kernel -- the decode stream for batches without a chunk.
//   combine_kernel, chunk_combine_kernel -- log-sum-exp merges of split ranges.
// Decode waves stream raw blocks and build 16x16x32 MFMA operands from the
// bytes; chunk tiles dequantize each 32-key step once into a shared LDS tile
// and run 16x16x32 MFMAs.  Quantized keys enter the MFMA as exact integer codes
// with their block scale applied in fp32.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "mab.h"

namespace {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // plain 16-byte vector (not HIP's uint4 struct)

// Loads through global-address-space pointers.  Every buffer the kernels
// read is device global memory; saying so makes the compiler emit global
// loads, which count only against the vector-memory counter (a generic
// pointer gives flat loads, which also count against the LDS counter, so that
// every wait for an LDS result would also wait for the loads in flight).
#define MAB_GLOBAL __attribute__((address_space(1)))
__device__ inline u32x4_t gload16_nt(const void* p) {
  return __builtin_nontemporal_load((const MAB_GLOBAL u32x4_t*)p);
}
__device__ inline int32_t gload_i32(const int32_t* p) { return *(const MAB_GLOBAL int32_t*)p; }
// Raw buffer resources: a wave-uniform base and a size in bytes; a load at an
// offset at or past the size returns zeros and touches no memory.  Word 3 is
// the gfx9 descriptor word for untyped 32-bit accesses.
constexpr int kCpolNt = 2;  // cache policy: non-temporal (streamed once)
__device__ inline __amdgpu_buffer_rsrc_t run_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
}
// Wait until at most N vector memory operations of this wave are in flight.
template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Debug mode (MAB_DEBUG=1 in the environment of the calling process): every
// page id read from the block table is checked against the pool; an id
// outside [0, num_pages) sets g_mab_debug_flag and page 0 is read or written
// instead, so the kernels stay inside the pools.  Otherwise ids are trusted.
// The kernels take it as a template flag: separate instantiations, so the
// normal ones carry no check.
__device__ int g_mab_debug_flag;
// The register form: an out-of-range id sets `bad`, which the caller reports
// once, after its loop.
__device__ inline int clamp_page(int page, int num_pages, int debug, int& bad) {
  const int out = debug & ((unsigned)page >= (unsigned)num_pages);
  bad |= out;
  return out ? 0 : page;
}
__device__ inline void report_bad_page(int bad) {
  if (bad) *(volatile int*)&g_mab_debug_flag = 1;
}
__device__ inline int checked_page(int page, int num_pages, int debug) {
  int bad = 0;
  page = clamp_page(page, num_pages, debug, bad);
  report_bad_page(bad);
  return page;
}

// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their maxima).
constexpr int kWaitVmcnt0 = 0x0F70;

constexpr int kDecodeWaves = 4;     // waves of a decode-kernel work-group (two work-groups per CU)
constexpr int kMixedWaves = 8;      // waves of a mixed-kernel work-group (one per CU)
constexpr int kStepKeys = 32;       // keys per stage / tile
constexpr int kMaxGroup = 8;        // query heads per KV head
constexpr int kMaxVerify = 16;      // sequences with at most this many rows run on the decode path
constexpr int kMaxSeqs = 4096;
constexpr int kMinWaveStages = 4;   // a decode work-group streams at least this many stages per wave
// Stages a decode wave has in flight beyond the one it computes on.  One is
// faster than two for every format (decode16 q8: 70.6 -> 61.4 us): the second
// register set of 16-byte loads crowds out the compute state at two waves per
// SIMD.
constexpr int kDecodeDepth = 1;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;  // a row keeps a stale max until it is 2^8 behind
// Decode weights P (up to 2^kRescaleSlack under the stale max) are multiplied
// by the V block scale in fp16.  A stage holding a V scale at or above this
// bound (fp16 bits; 128.0) takes the exact running max instead (P <= 1), so
// P * scale stays below 2^15 in every stage whatever the scale (at most 9360,
// the 4-bit scale of a block at the fp16 maximum).
constexpr uint16_t kBigVScaleBits = 0x5800u;
constexpr float kDecodeMaxFloor = -1e30f;  // initial running max of a decode slot (log2 units)

template <int F> struct Fmt;
template <> struct Fmt<MAB_KV_Q8> { static constexpr int kBytes = 34; static constexpr int kQmax = 127; };
template <> struct Fmt<MAB_KV_Q4> { static constexpr int kBytes = 18; static constexpr int kQmax = 7; };
// the unquantized mode: a block is its 32 values as fp16, no scale
template <> struct Fmt<MAB_KV_F16> { static constexpr int kBytes = 64; static constexpr int kQmax = 0; };
// offset of a block's values (after the scale of the quantized formats)
template <int F> constexpr int kPayload = F == MAB_KV_F16 ? 0 : 2;

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A chunk tile is one work-group of kMixedWaves = 8 waves, each serving 32
// rows of one query head: H heads of the group (the largest of 4, 2, 1 that
// divides G) times 256/H rows.  Its K/V steps are dequantized once for all.
__host__ __device__ inline int chunk_heads(int group) { return group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1; }
__host__ __device__ inline int chunk_rows(int group) { return 32 * kMixedWaves / chunk_heads(group); }

// Rows of a sequence with q_len <= kMaxVerify (decode rows and short verify
// rows) run on the decode path, in sub-rows of at most T consecutive rows
// whose (row, head) pairs fill the MFMA slots of a decode wave: one group of
// 16 slots (T = 16/G), or, for a sequence with more than 16/G rows over
// quantized pools (`wide`), two groups of 16 that share every stage read
// (T = 32/G).  Sub-row i holds rows [i*T, min(q_len, (i+1)*T)) and streams
// the keys its last row sees.  Longer sequences are prefill chunks.
__host__ __device__ inline bool is_chunk(int q_len) { return q_len > kMaxVerify; }
__host__ __device__ inline int dec_tokens(int q_len, int group, bool wide) {
  return wide && q_len > 16 / group ? 32 / group : 16 / group;
}
__host__ __device__ inline int dec_subrows(int q_len, int group, bool wide) {
  const int t = dec_tokens(q_len, group, wide);
  return (q_len + t - 1) / t;
}

// A prefill chunk: ceil(q_len/rows) row tiles x Hkv x G/H head groups, each
// cut into a number of key splits (one work item per split).  A decode
// sub-row: Hkv segments of ceil(ctx/32) stages each in the decode stream, ctx
// the keys its last row sees.
__host__ __device__ inline int chunk_tiles(int q_len, int hkv, int group) {
  return ceil_div(q_len, chunk_rows(group)) * hkv * (group / chunk_heads(group));
}
// Tile t of a chunk sequence with n_qt row tiles, n_hp head groups and hkv
// KV heads: row tile qt, head group hp, KV head g; a tile's F key splits are
// work items t*F .. t*F+F-1.  The row tile varies slowest and runs last
// first: a later row tile sees more keys, and work items start in grid order
// as work-groups free, so the longest items start first and the last to
// start are short.  The items of one row tile (all head groups, KV heads and
// splits, equally long) are consecutive, so the work-groups, dealt
// round-robin over the eight XCDs, give each XCD an equal share; the KV head
// varies fastest, so an XCD sees the same few (KV head, key split) ranges in
// every row tile and its items share their K/V bytes in its L2.
struct ChunkTileCoord { int qt, hp, g; };
__host__ __device__ inline ChunkTileCoord chunk_tile_coord(int t, int n_qt, int n_hp, int hkv) {
  const int u = t / hkv;
  return ChunkTileCoord{n_qt - 1 - u / n_hp, u % n_hp, t % hkv};
}
__host__ __device__ inline int dec_stages(int ctx) { return ceil_div(ctx, kStepKeys); }
// Units a decode segment takes in the decode stream: its stages, or, for
// batches with MAB_BATCH_INVARIANT (piece = stages per piece), its stages
// rounded up to whole pieces, so that every segment starts on a piece
// boundary and the pieces of one range per wave are cut from the segment's
// own first key.  The padding units hold no work.
constexpr int kInvariantPiece = MAB_INVARIANT_PIECE_KEYS / kStepKeys;
static_assert(MAB_INVARIANT_PIECE_KEYS % kStepKeys == 0, "whole stages per invariant piece");
__host__ __device__ inline int dec_units_of(int ctx, int piece) {
  const int n = dec_stages(ctx);
  return piece > 0 ? ceil_div(n, piece) * piece : n;
}

// Key splits per tile of a chunk sequence: the F in 1..8 whose tiles*F work
// items fill whole rounds of `slots` resident work-groups best (the smallest
// such F).  It depends only on the sequence's own tile count and the device,
// so a chunk row's arithmetic is the same whatever shares the batch.
constexpr int kMaxChunkSplit = 8;
__host__ __device__ inline int chunk_split(int tiles, int slots) {
  int best = 1;
  int64_t best_num = 0, best_den = 1;  // efficiency = num / den
  for (int f = 1; f <= kMaxChunkSplit; ++f) {
    const int64_t items = (int64_t)tiles * f;
    const int64_t den = ((items + slots - 1) / slots) * slots;
    if (items * best_den > best_num * den) {
      best = f;
      best_num = items;
      best_den = den;
    }
  }
  return best;
}

__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Where a decode segment's results went: its first piece's partial slot, the
// decode worker (wave) that ran that piece, the number of pieces (1: the
// output was written directly) and the segment's first output row-head.
struct DirEntry {
  int slot, wg, n, rh0;
};

// Workspace: decode partials (slot = worker * pmax + piece; o fp32
// [slot][P][D], (m, l) fp32 pairs [slot][P], P the (row, head) slots of a
// decode sub-row), chunk partials of split tiles
// (o fp32 [item][G][rows][D], (m, l) [item][G][rows]), one directory entry per
// decode segment, and the launch-order tables for batches too large for the
// kernel arguments.  Nothing needs initialising: every entry read is written
// first in the same call.
struct WsLayout {
  int64_t o_off, ml_off, cho_off, chml_off, dir_off, tab_off, total;
};

__host__ __device__ inline WsLayout ws_layout(int64_t n_slots, int per_slot, int head_dim, int64_t n_chunk_rows,
                                              int64_t n_dec_segs, int64_t tab_ints) {
  WsLayout w;  // per_slot: (row, head) pairs of a decode partial
  w.o_off = 0;
  w.ml_off = align256(w.o_off + n_slots * per_slot * head_dim * 4);
  w.cho_off = align256(w.ml_off + n_slots * per_slot * 8);
  w.chml_off = align256(w.cho_off + n_chunk_rows * head_dim * 4);
  w.dir_off = align256(w.chml_off + n_chunk_rows * 8);
  w.tab_off = align256(w.dir_off + n_dec_segs * (int64_t)sizeof(DirEntry));
  w.total = align256(w.tab_off + tab_ints * 4);
  return w;
}

// ---------------------------------------------------------------------------
// Append: one thread encodes one 32-value block.
// ---------------------------------------------------------------------------

__device__ inline int find_seq(const int32_t* __restrict__ q_start, int num_seqs, int row) {
  int lo = 0, hi = num_seqs - 1;  // largest s with q_start[s] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (q_start[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int F>
__device__ inline void encode_block(const half_t* __restrict__ x, uint8_t* __restrict__ dst) {
  if constexpr (F == MAB_KV_F16) {  // the values themselves (blocks of 64 bytes, 16-byte aligned)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      reinterpret_cast<half8_t*>(dst)[i] = reinterpret_cast<const half8_t*>(x)[i];
  } else {
    constexpr int Q = Fmt<F>::kQmax;
    float xf[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half8_t v = *reinterpret_cast<const half8_t*>(x + 8 * i);
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[8 * i + e] = (float)v[e];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(xf[i]));
    int code[32];
    uint16_t dbits = 0;
    if (amax > 0.f) {
      const float s = amax / (float)Q;                 // IEEE binary32 divide
      const half_t d = (half_t)s;                      // RNE, fp16 subnormals kept
      dbits = __builtin_bit_cast(uint16_t, d);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        float r = rintf(xf[i] / s);                    // half to even
        r = fminf(fmaxf(r, -(float)Q), (float)Q);
        code[i] = (int)r;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) code[i] = 0;
    }
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);  // blocks start on even bytes
    d16[0] = dbits;
    if constexpr (F == MAB_KV_Q8) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        d16[1 + i] = (uint16_t)((code[2 * i] & 0xFF) | ((code[2 * i + 1] & 0xFF) << 8));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int b0 = (code[4 * i] & 0xF) | ((code[4 * i + 1] & 0xF) << 4);
        const int b1 = (code[4 * i + 2] & 0xF) | ((code[4 * i + 3] & 0xF) << 4);
        d16[1 + i] = (uint16_t)(b0 | (b1 << 8));
      }
    }
  }
}

template <int KF, int VF, bool DBG>
__global__ void __launch_bounds__(256)
append_kernel(const half_t* __restrict__ k_new, const half_t* __restrict__ v_new,
              uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
              const int32_t* __restrict__ q_start, const int32_t* __restrict__ prefix_len,
              const int32_t* __restrict__ block_table, int num_seqs, int num_rows,
              int max_pages, int hkv, int head_dim, int page_size, int num_pages) {
  const int nb = head_dim / 32;
  const int64_t per_side = (int64_t)num_rows * hkv * nb;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= 2 * per_side) return;
  const bool is_v = tid >= per_side;
  const int64_t u = is_v ? tid - per_side : tid;
  const int b = (int)(u % nb);
  const int g = (int)((u / nb) % hkv);
  const int row = (int)(u / ((int64_t)nb * hkv));
  const int s = find_seq(q_start, num_seqs, row);
  const int pos = prefix_len[s] + (row - q_start[s]);
  const int page = checked_page(block_table[(int64_t)s * max_pages + pos / page_size], num_pages, DBG);
  const int slot = pos % page_size;
  const int64_t tok = ((int64_t)page * hkv + g) * page_size + slot;
  const half_t* src = (is_v ? v_new : k_new) + ((int64_t)row * hkv + g) * head_dim + 32 * b;
  if (is_v) encode_block<VF>(src, v_pool + (tok * nb + b) * Fmt<VF>::kBytes);
  else encode_block<KF>(src, k_pool + (tok * nb + b) * Fmt<KF>::kBytes);
}

// ---------------------------------------------------------------------------
// Attention: shared pieces
// ---------------------------------------------------------------------------

struct ItemCtx {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* bt_row;  // block-table row of the sequence
  int hkv, g, page_size;
};

// Online-softmax state of one decode wave.  The 16 MFMA slots are the (row,
// head) pairs of a decode sub-row (for a decode row, the G query heads of the
// KV head); lane l serves slot l%16, and the four lanes of a slot hold
// different keys of S^T and different dims of O^T.
template <int NB>
struct Group {
  half8_t q[NB];          // Q^T operand: slot l%16, dims 32b + 8(l/16) + [0,8)
  float4_t o[2 * NB];     // O^T tile t of block t/2: slot l%16, rows 4(l/16) + [0,4), row r being value
                          // 2r + t%2 of the block; V codes taken with their bias
  float4_t vb[NB];        // per block: sum over keys of the P * V-scale weights (the bias correction of o)
  float vs[NB];           // the same sums, lane-partial (two-group waves: the MFMA form costs 12 more registers)
  float m, l;             // running max (log2 units) and lane-partial sum
  int limit;              // last key position visible to the slot (-1: none)
};

// V codes enter the PV products as fp16 integers carrying the bias of the
// magic-number conversion (1152 + code for 8-bit codes, 1032 + code for
// 4-bit codes); o is corrected once at the end by bias * (sum of weights).
template <int F> struct VBias;
template <> struct VBias<MAB_KV_Q8> { static constexpr float kBias = 1152.f; };
template <> struct VBias<MAB_KV_Q4> { static constexpr float kBias = 1032.f; };
template <> struct VBias<MAB_KV_F16> { static constexpr float kBias = 0.f; };  // the values themselves


template <int NB>
__device__ inline void group_init(Group<NB>& gr, const half_t* qrow, int limit, int lane) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (qrow) gr.q[b] = *reinterpret_cast<const half8_t*>(qrow + 32 * b + 8 * (lane >> 4));
    else gr.q[b] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }
#pragma unroll
  for (int t = 0; t < 2 * NB; ++t) gr.o[t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < NB; ++b) gr.vb[b] = float4_t{0.f, 0.f, 0.f, 0.f};
  gr.m = -INFINITY;
  gr.l = 0.f;
  gr.limit = qrow ? limit : -1;
}

// Element order (0,2,4,6,1,3,5,7): 4-bit codes are unpacked low nibbles first.
__device__ inline half8_t nibble_order(half8_t q) {
  return half8_t{q[0], q[2], q[4], q[6], q[1], q[3], q[5], q[7]};
}

// Max over lanes l and l^16 (l^32): the row-swap instructions put the values
// of both lanes of a pair into the two results, in either order.
__device__ inline float max_xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ inline float max_xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// ---------------------------------------------------------------------------
// Raw stage: the bytes of 32 keys of one KV head, K then V, each as two
// 16-key runs copied whole (a run never crosses a page: page_size % 16 == 0).
// Decode waves build MFMA operands from it directly; chunk tiles dequantize it.
// ---------------------------------------------------------------------------

template <int NB, int KF, int VF>
struct DecLayout {
  static constexpr int kBK = Fmt<KF>::kBytes, kBV = Fmt<VF>::kBytes;
  static constexpr int kRecK = NB * kBK, kRecV = NB * kBV;   // bytes per key of one KV head
  static constexpr int kKBytes = kStepKeys * kRecK, kVBytes = kStepKeys * kRecV;
  static constexpr int kChunksK = kKBytes / 16, kChunksV = kVBytes / 16;
  static constexpr int kChunks = kChunksK + kChunksV;
  static constexpr int kLoads = (kChunks + 63) / 64;          // 16-byte loads per lane per stage
  static constexpr int kKOff = 0;
  static constexpr int kVOff = kKBytes;
  static constexpr int kRawBytes = kLoads * 1024 + 16;        // one stage buffer: tail lanes + over-read pad
  static constexpr int kSKOff = kRawBytes;                    // float [NB][32]: K scale * c
  static constexpr int kSVOff = kSKOff + NB * kStepKeys * 4;  // half  [NB][32]: V scale
  static constexpr int kWaveBytes = kSVOff + NB * kStepKeys * 2;
  // kernels with wide verify pieces (quantized pools): a second stage buffer
  // after the scales, for the two-buffer ring of those pieces
  static constexpr bool kWideOk = KF != MAB_KV_F16 && VF != MAB_KV_F16;
  static constexpr int kWideBytes = kWaveBytes + kRawBytes;
  // The stage as four 16-key runs of 16-byte chunks, each contiguous in its
  // pool: K of keys 0-15, K of keys 16-31, V of keys 0-15, V of keys 16-31
  // (a run of 16 keys holds kRecK, resp. kRecV, chunks).  Run q covers
  // chunks [run_lo(q), run_lo(q+1)); the last run also takes the lanes past
  // the last chunk (they read zeros).  run_load_issues: the loads of a stage
  // loaded run by run (one per run that meets each 64-chunk load).
  static constexpr int run_lo(int q) {
    return q == 0 ? 0 : q == 1 ? kRecK : q == 2 ? 2 * kRecK : q == 3 ? 2 * kRecK + kRecV : 64 * kLoads;
  }
  static constexpr bool run_meets(int q, int i) { return run_lo(q) < 64 * i + 64 && run_lo(q + 1) > 64 * i; }
  static constexpr int run_load_issues() {
    int n = 0;
    for (int i = 0; i < kLoads; ++i)
      for (int q = 0; q < 4; ++q) n += run_meets(q, i) ? 1 : 0;
    return n;
  }
  static_assert(kKBytes % 16 == 0 && kVBytes % 16 == 0 && kWaveBytes % 16 == 0, "alignment");
};

__device__ inline uint32_t lds_u32(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}

// 8 int8 codes (two dwords, little-endian) as exact fp16 integers
// (magic-number conversion: 0x6400|(c^0x80) is 1152 + c in fp16).
__device__ inline half8_t codes8_q8(uint32_t w0, uint32_t w1) {
  w0 ^= 0x80808080u;
  w1 ^= 0x80808080u;
  const half2_t bias = {(half_t)-1152.f, (half_t)-1152.f};
  half2_t h[4];
  h[0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u)) + bias;
  h[1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u)) + bias;
  h[2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u)) + bias;
  h[3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u)) + bias;
  return half8_t{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
}

// Four bytes holding offset-8 nibbles (one value per byte, 0..15) as fp16 v - 8.
__device__ inline half4_t nib4(uint32_t v) {
  const half2_t bias = {(half_t)-1032.f, (half_t)-1032.f};
  const half2_t a = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, v, 0x04010400u)) + bias;
  const half2_t b = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, v, 0x04030402u)) + bias;
  return half4_t{a[0], a[1], b[0], b[1]};
}

// 8 two's-complement nibbles (one dword), returned in the element order
// (0,2,4,6,1,3,5,7) of the 8 values they encode.
__device__ inline half8_t codes8_q4(uint32_t w) {
  w ^= 0x88888888u;  // nibble + 8
  const half4_t lo = nib4(w & 0x0F0F0F0Fu), hi = nib4((w >> 4) & 0x0F0F0F0Fu);
  return half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 8 int8 codes starting at an even byte offset, as exact fp16 integers.
__device__ inline half8_t lds_codes8_q8(const uint8_t* base, int off) {
  const int a = off & ~3, sh = off & 3;
  const uint32_t d0 = lds_u32(base, a), d1 = lds_u32(base, a + 4), d2 = lds_u32(base, a + 8);
  return codes8_q8(__builtin_amdgcn_alignbyte(d1, d0, sh), __builtin_amdgcn_alignbyte(d2, d1, sh));
}

// 8 two's-complement nibbles starting at an even byte offset, returned in the
// element order (0,2,4,6,1,3,5,7) of the 8 values they encode.
__device__ inline half8_t lds_codes8_q4(const uint8_t* base, int off) {
  const int a = off & ~3, sh = off & 3;
  const uint32_t d0 = lds_u32(base, a), d1 = lds_u32(base, a + 4);
  return codes8_q4(__builtin_amdgcn_alignbyte(d1, d0, sh));
}

// Values 2v and 2v+1 (within block) of two keys whose block payloads start at
// byte offsets o0, o1: p0 = (value 2v of key 0, of key 1), p1 = (value 2v+1 of
// each), as fp16 pairs of exact integers offset by VBias<F>::kBias (1152 +
// code, or 1032 + code for 4-bit codes), or the fp16 values themselves.  The
// two values of a key sit in one 2-byte word (8-bit codes), one byte (4-bit
// codes) or one 4-byte word (fp16), so one read per key serves both.  Row n
// of a block's two 16-row V^T tiles t2 is value 2n + t2.
template <int F>
__device__ inline void lds_value_pairs_biased(const uint8_t* base, int o0, int o1, int v, half2_t& p0, half2_t& p1) {
  if constexpr (F == MAB_KV_F16) {
    const uint32_t a = *reinterpret_cast<const uint32_t*>(base + o0 + 4 * v);
    const uint32_t b = *reinterpret_cast<const uint32_t*>(base + o1 + 4 * v);
    p0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(b, a, 0x05040100u));
    p1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(b, a, 0x07060302u));
  } else if constexpr (F == MAB_KV_Q8) {
    uint32_t w = (uint32_t)*reinterpret_cast<const uint16_t*>(base + o0 + 2 * v) |
                 ((uint32_t)*reinterpret_cast<const uint16_t*>(base + o1 + 2 * v) << 16);
    w ^= 0x80808080u;  // bytes: key 0 value 2v, 2v+1, key 1 value 2v, 2v+1; 0x64xx is 1152 + code
    p0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, w, 0x04020400u));
    p1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, w, 0x04030401u));
  } else {  // 4-bit codes: value 2v in the low nibble of byte v, 2v+1 in the high nibble
    const uint32_t w = (uint32_t)base[o0 + v] | ((uint32_t)base[o1 + v] << 16);
    p0 = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) ^ 0x64086408u);
    p1 = __builtin_bit_cast(half2_t, ((w >> 4) & 0x000F000Fu) ^ 0x64086408u);
  }
}

// p, which holds the same value in every lane, as a value the compiler keeps
// in scalar registers.
template <typename T>
__device__ inline const T* wave_uniform(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

template <int NB, int KF, int VF>
struct DecWave {
  using L = DecLayout<NB, KF, VF>;
  u32x4_t r[L::kLoads];  // the next stage's raw bytes, in flight

  // The loads of a stage whose 32 keys lie in one page (page_size a multiple
  // of 32): its K bytes and its V bytes are each one contiguous run, so every
  // load is a scalar run base plus a lane offset that does not change from
  // stage to stage (16*lane + 1024*i, clamped on the last load); only the
  // load that straddles the K/V boundary picks its base per lane.
  __device__ __attribute__((always_inline)) void load_page(const ItemCtx& c, int kbase, int page, int lane) {
    const int64_t tok = ((int64_t)page * c.hkv + c.g) * c.page_size + kbase % c.page_size;
    const uint8_t* kr = wave_uniform(c.k_pool + tok * L::kRecK);
    const uint8_t* vr = wave_uniform(c.v_pool + tok * L::kRecV);
    const uint32_t lo = 16u * (uint32_t)lane;
#pragma clang loop unroll(full)
    for (int i = 0; i < L::kLoads; ++i) {
      const uint8_t* src;
      if (64 * i + 63 < L::kChunksK) {
        src = kr + (lo + 1024u * i);
      } else if (64 * i >= L::kChunksK) {
        const int c0 = 64 * i - L::kChunksK;
        if (64 * i + 63 < L::kChunks) src = vr + (lo + 16u * c0);
        else src = vr + 16u * (uint32_t)min(lane + c0, L::kChunksV - 1);  // lanes past the last chunk re-read it
      } else {
        const int ch = lane + 64 * i;
        src = ch < L::kChunksK ? kr + 16u * (uint32_t)ch : vr + 16u * (uint32_t)(ch - L::kChunksK);
      }
      r[i] = gload16_nt(src);  // streamed once
    }
  }

  // Issue the loads of keys [kbase, kbase+32) of KV head c.g: two 16-key runs,
  // each inside one page (ids page0, page1).  A run at or past kend re-reads
  // run 0 instead (its keys are masked), and lanes past the last chunk re-read
  // the last chunk, so every lane loads valid memory without branching.
  __device__ __attribute__((always_inline)) void load(const ItemCtx& c, int kbase, int kend, int page0, int page1, int lane) {
    const int ps = c.page_size;
    const int key1 = kbase + 16;
    const int64_t tok0 = ((int64_t)page0 * c.hkv + c.g) * ps + kbase % ps;
    const int64_t tok1 = key1 < kend ? ((int64_t)page1 * c.hkv + c.g) * ps + key1 % ps : tok0;
    const uint8_t* k0 = c.k_pool + tok0 * L::kRecK;
    const uint8_t* k1 = c.k_pool + tok1 * L::kRecK;
    const uint8_t* v0 = c.v_pool + tok0 * L::kRecV;
    const uint8_t* v1 = c.v_pool + tok1 * L::kRecV;
#pragma clang loop unroll(full)
    for (int i = 0; i < L::kLoads; ++i) {
      const int ch = lane + 64 * i;
      const uint8_t* src;
      if (64 * i + 63 < L::kChunksK) {          // all lanes in the K region
        src = ch < L::kRecK ? k0 + 16 * ch : k1 + 16 * (ch - L::kRecK);
      } else if (64 * i >= L::kChunksK) {       // all lanes in the V region
        const int cv = min(ch - L::kChunksK, L::kChunksV - 1);
        src = cv < L::kRecV ? v0 + 16 * cv : v1 + 16 * (cv - L::kRecV);
      } else {                                  // the boundary load
        const int cv = ch - L::kChunksK;
        src = ch < L::kRecK ? k0 + 16 * ch
            : ch < L::kChunksK ? k1 + 16 * (ch - L::kRecK)
            : cv < L::kRecV ? v0 + 16 * cv : v1 + 16 * (cv - L::kRecV);
      }
      r[i] = gload16_nt(src);  // streamed once
    }
  }

  // Copy the stage into LDS (lanes past the last chunk land in the tail pad).
  __device__ __attribute__((always_inline)) void store(uint8_t* w, int lane) {
#pragma clang loop unroll(full)
    for (int i = 0; i < L::kLoads; ++i) *reinterpret_cast<u32x4_t*>(w + 16 * (lane + 64 * i)) = r[i];
  }
};

// One buffer load of a stage loaded run by run: load I (chunks 64I..64I+63)
// for the lanes whose chunk lies in run Q.  The byte of the run at lane 0 of
// the load goes in the instruction's offset field when it is not negative
// (a run that starts inside the load: into the lane offset; the lanes before
// the run start are off).  The offset field moves the LDS address as well as
// the memory address, so the LDS base given is that much lower.
template <int NB, int KF, int VF, int I, int Q>
__device__ __attribute__((always_inline)) inline void dec_run_load(const __amdgpu_buffer_rsrc_t (&r)[4], uint32_t voff,
                                                                   uint8_t* buf, int lane) {
  using L = DecLayout<NB, KF, VF>;
  if constexpr (L::run_meets(Q, I)) {
    constexpr int shift = 1024 * I - 16 * L::run_lo(Q);
    static_assert(shift < 4096, "the offset field holds 12 bits");
    constexpr bool whole = L::run_lo(Q) <= 64 * I && L::run_lo(Q + 1) >= 64 * I + 64;
    const int ch = lane + 64 * I;
    using lds_t = __attribute__((address_space(3))) void*;
    if (whole || (ch >= L::run_lo(Q) && ch < L::run_lo(Q + 1))) {
      if constexpr (shift >= 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r[Q], (lds_t)(buf + 1024 * I - shift), 16, voff, 0, shift, kCpolNt);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r[Q], (lds_t)(buf + 1024 * I), 16, voff + shift, 0, 0, kCpolNt);
    }
  }
}

template <int NB, int KF, int VF, int... IQ>
__device__ __attribute__((always_inline)) inline void dec_run_loads(const __amdgpu_buffer_rsrc_t (&r)[4], uint32_t voff,
                                                                    uint8_t* buf, int lane,
                                                                    std::integer_sequence<int, IQ...>) {
  (dec_run_load<NB, KF, VF, IQ / 4, IQ % 4>(r, voff, buf, lane), ...);
}

// Loads the 32 keys of a stage straight into the LDS stage buffer buf, run
// by run (run bases k0, k1, v0, v1; run1 false: keys 16-31 are past the
// piece and read as zeros): chunk c lands at buf + 16c, as the register form
// stores it.  Issues L::run_load_issues() buffer loads; a load that meets two
// runs is issued once per run, each for its own lanes.  Each run's resource
// ends where the run ends, so lanes past it (the tail, or a run that is off)
// read zeros.
template <int NB, int KF, int VF>
__device__ __attribute__((always_inline)) inline void dec_stage_to_lds(uint8_t* buf, const uint8_t* k0,
                                                                       const uint8_t* k1, const uint8_t* v0,
                                                                       const uint8_t* v1, bool run1, int lane) {
  using L = DecLayout<NB, KF, VF>;
  // the bases and sizes are wave-uniform: say so, so that the resources live
  // in scalar registers
  const int on1 = __builtin_amdgcn_readfirstlane(run1 ? 1 : 0);
  const __amdgpu_buffer_rsrc_t r[4] = {
      run_rsrc(wave_uniform(k0), 16 * L::kRecK), run_rsrc(wave_uniform(k1), on1 * 16 * L::kRecK),
      run_rsrc(wave_uniform(v0), 16 * L::kRecV), run_rsrc(wave_uniform(v1), on1 * 16 * L::kRecV)};
  dec_run_loads<NB, KF, VF>(r, 16u * (uint32_t)lane, buf, lane, std::make_integer_sequence<int, 4 * L::kLoads>{});
}

// Pulls the K and V block scales of the stage in LDS (stage buffer raw) into
// the compact arrays of the wave area w:
// K scales as fp32 times c = sm_scale*log2(e), V scales as fp16, both [block][key].
// Keys at or past kend get scale 0, so their (possibly NaN) bytes never reach
// a sum: their logits become exactly 0 before masking and their P*scale 0.
// Returns (wave-uniform) whether some V scale of the stage is at or above
// kBigVScaleBits.
template <int NB, int KF, int VF>
__device__ inline bool dec_scales(const uint8_t* raw, uint8_t* w, int lane, float zc, int nvalid) {
  using L = DecLayout<NB, KF, VF>;
  bool big = false;
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const int idx = lane + 64 * q;            // NB*64 = 2*32*NB entries: K first, then V
    const bool isv = q >= NB / 2;
    const int m = isv ? idx - 32 * NB : idx;
    const int b = m / kStepKeys, key = m % kStepKeys;
    const bool ok = key < nvalid;
    if (!isv) {
      float d = 1.f;  // the unquantized format has no scale
      if constexpr (KF != MAB_KV_F16)
        d = (float)__builtin_bit_cast(half_t, *reinterpret_cast<const uint16_t*>(raw + L::kKOff + key * L::kRecK +
                                                                                  b * L::kBK));
      reinterpret_cast<float*>(w + L::kSKOff)[m] = ok ? d * zc : 0.f;
    } else {
      uint16_t bits = 0x3C00u;  // fp16 1.0
      if constexpr (VF != MAB_KV_F16)
        bits = *reinterpret_cast<const uint16_t*>(raw + L::kVOff + key * L::kRecV + b * L::kBV);
      reinterpret_cast<uint16_t*>(w + L::kSVOff)[m] = ok ? bits : (uint16_t)0;
      big |= ok && bits >= kBigVScaleBits;  // scales are non-negative: bit order is value order
    }
  }
  return __any(big);
}

// One 32-key stage of a decode wave over NG slot groups (NG = 2: a wide
// verify sub-row; both groups share the stage's K and V operands): S^T = K Q^T
// on integer codes per block, fp32 block scales, online softmax with a stale
// max (rescaled only when the running max grows by more than 2^kRescaleSlack;
// by any amount in a stage with a large V scale, `big_v`), then O^T += V^T
// (P * V scale) with P rounded to fp16 once and multiplied by the fp16 V scale
// of each block.  The normaliser sums the same fp16 P.  The V codes enter with
// the bias of their conversion; the sum of each block's weights (an MFMA
// against ones) removes it at the end.  `raw`: the stage's bytes; `w`: the
// wave area holding the compact scales.  `tail`: the stage holds keys at or
// past kend, or past the limit of some slot (masked per slot).
template <int NB, int KF, int VF, int NG>
__device__ inline void dec_compute(Group<NB> (&gr)[NG], const uint8_t* raw, const uint8_t* w, int kbase, int kend,
                                   bool tail, bool big_v, int lane) {
  using L = DecLayout<NB, KF, VF>;
  const int j = lane >> 4, n = lane & 15;
  float4_t s[NG][2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int k = 0; k < NG; ++k) s[k][kt] = float4_t{0.f, 0.f, 0.f, 0.f};
    const int rec = (16 * kt + n) * L::kRecK;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      half8_t kc;
      if constexpr (KF == MAB_KV_F16) kc = *reinterpret_cast<const half8_t*>(raw + L::kKOff + rec + b * L::kBK + 16 * j);
      else if constexpr (KF == MAB_KV_Q8) kc = lds_codes8_q8(raw + L::kKOff, rec + b * L::kBK + 2 + 8 * j);
      else kc = lds_codes8_q4(raw + L::kKOff, rec + b * L::kBK + 2 + 4 * j);
      const float4_t kd = *reinterpret_cast<const float4_t*>(w + L::kSKOff + 4 * (b * kStepKeys + 16 * kt + 4 * j));
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        const float4_t pb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc, gr[k].q[b], float4_t{0.f, 0.f, 0.f, 0.f},
                                                                   0, 0, 0);
        s[k][kt] += kd * pb;
      }
    }
  }
  half8_t ph[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    Group<NB>& g = gr[k];
    if (tail) {
      // keys visible to this lane's slot in the stage: below kend and at most g.limit
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kbase + 16 * kt + 4 * j + i >= min(kend, g.limit + 1)) s[k][kt][i] = -INFINITY;
    }
    // the slot's max grows past the threshold only if one of its lanes' values
    // does: the lane-swap reduction runs only then (rarely after the first
    // stages)
    const float lmx = fmaxf(fmaxf(fmaxf(s[k][0][0], s[k][0][1]), fmaxf(s[k][0][2], s[k][0][3])),
                            fmaxf(fmaxf(s[k][1][0], s[k][1][1]), fmaxf(s[k][1][2], s[k][1][3])));
    const float thr = g.m + (big_v ? 0.f : kRescaleSlack);  // -inf for the first keys (m = -inf)
    if (__any(lmx > thr)) {
      const float mx = max_xor32(max_xor16(lmx));
      const bool grow = mx > thr;
      const float m_new = grow ? mx : g.m;
      const float alpha = grow ? __builtin_amdgcn_exp2f(g.m - m_new) : 1.f;  // 0 when m was -inf
#pragma unroll
      for (int t = 0; t < 2 * NB; ++t) g.o[t] *= alpha;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if constexpr (NG == 1) g.vb[b] *= alpha;
        else g.vs[b] *= alpha;
      }
      g.l *= alpha;
      g.m = m_new;
    }
    float p[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[4 * kt + i] = __builtin_amdgcn_exp2f(s[k][kt][i] - g.m);  // <= 2^kRescaleSlack (1 if big_v); masked 0
    // P as fp16 in the key order of the PV operand: 4j+[0,4) then 16+4j+[0,4)
    ph[k] = half8_t{(half_t)p[0], (half_t)p[1], (half_t)p[2], (half_t)p[3],
                    (half_t)p[4], (half_t)p[5], (half_t)p[6], (half_t)p[7]};
    // the normaliser sums the fp16 weights that the PV products use
    const half2_t one2 = half2_t{(half_t)1.f, (half_t)1.f};
    float psum = __builtin_amdgcn_fdot2(half2_t{ph[k][0], ph[k][1]}, one2, 0.f, false);
    psum = __builtin_amdgcn_fdot2(half2_t{ph[k][2], ph[k][3]}, one2, psum, false);
    psum = __builtin_amdgcn_fdot2(half2_t{ph[k][4], ph[k][5]}, one2, psum, false);
    psum = __builtin_amdgcn_fdot2(half2_t{ph[k][6], ph[k][7]}, one2, psum, false);
    g.l += psum;
  }
  const half_t* sv = reinterpret_cast<const half_t*>(w + L::kSVOff);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const half4_t s0 = *reinterpret_cast<const half4_t*>(sv + b * kStepKeys + 4 * j);
    const half4_t s1 = *reinterpret_cast<const half4_t*>(sv + b * kStepKeys + 16 + 4 * j);
    const half8_t svb = half8_t{s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    half8_t pf[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      pf[k] = ph[k] * svb;
      if constexpr (VBias<VF>::kBias != 0.f) {  // sum of the weights
        if constexpr (NG == 1) {
          const half8_t ones = half8_t{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
          gr[k].vb[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[k], gr[k].vb[b], 0, 0, 0);
        } else {
          const half2_t one2 = half2_t{(half_t)1.f, (half_t)1.f};
          float t = gr[k].vs[b];
#pragma unroll
          for (int e = 0; e < 4; ++e) t = __builtin_amdgcn_fdot2(half2_t{pf[k][2 * e], pf[k][2 * e + 1]}, one2, t, false);
          gr[k].vs[b] = t;
        }
      }
    }
    // the block's two V^T tiles: row n of tile t2 is value 2n + t2 of the block
    half2_t vp[2][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ka = (e < 2) ? 4 * j + 2 * e : 16 + 4 * j + 2 * (e - 2);
      lds_value_pairs_biased<VF>(raw + L::kVOff, ka * L::kRecV + b * L::kBV + kPayload<VF>,
                                 (ka + 1) * L::kRecV + b * L::kBV + kPayload<VF>, n, vp[0][e], vp[1][e]);
      if constexpr (VF == MAB_KV_F16) {
        // f16 values of keys past the range are whatever the pool holds there
        // (possibly NaN): zero them, as their weight is zero
        if (tail) {
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            if (kbase + ka >= kend) vp[t2][e][0] = (half_t)0.f;
            if (kbase + ka + 1 >= kend) vp[t2][e][1] = (half_t)0.f;
          }
        }
      }
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const half8_t vc = half8_t{vp[t2][0][0], vp[t2][0][1], vp[t2][1][0], vp[t2][1][1],
                                 vp[t2][2][0], vp[t2][2][1], vp[t2][3][0], vp[t2][3][1]};
#pragma unroll
      for (int k = 0; k < NG; ++k)
        gr[k].o[2 * b + t2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vc, pf[k], gr[k].o[2 * b + t2], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk path.  Every 32-key step is dequantized once into a shared LDS tile
// (K as exact integer codes with fp32 block scales times sm_scale*log2(e), V
// as fp16 values, both [key][dim]); tiles are double buffered.  Each wave
// serves one query head and 32 rows as two 16-row tiles of 16x16x32 MFMAs:
// S^T = K Q^T per 32-dim block on integer codes, scaled per key in fp32 and
// taken relative to the row's running max, then O^T += V^T P^T with the V^T
// operand read by LDS transpose reads.  A step: dequantize step s+1 from
// registers into the other tile, issue the global loads of step s+3, compute
// step s, one barrier.
// ---------------------------------------------------------------------------

template <int NB>
struct ChunkTile {
  static constexpr int kD = 32 * NB;
  static constexpr int kStride = kD + 8;   // halves per key row: rows 16 bytes apart modulo 256
  half_t k[kStepKeys * kStride];           // K codes (exact integers)
  half_t v[kStepKeys * kStride];           // fp16(V code * scale)
  float kd[NB * kStepKeys];                // K block scale times c = sm_scale*log2(e), [block][key]
};

// Value index (0..31 within a block) held at position p of a block's LDS row
// segment.  4-bit codes are unpacked low nibbles first, so each group of 8
// values is stored in the order (0,2,4,6,1,3,5,7); Q and the output follow suit.
template <int F>
__device__ inline int value_of_slot(int p) {
  if constexpr (F != MAB_KV_Q4) return p;
  else return (p & ~7) | ((p & 3) << 1) | ((p & 4) >> 2);
}

// The raw bytes of one dequant unit (the scale and 32 codes of one block of
// one key of K or V), loaded as dwords from the 4-byte-aligned address at or
// below the block (the block starts at byte 0 or 2 of w).  The dwords of a
// 4-bit block sit where those of an 8-bit block do (its last one in w[8]),
// so that a wave's K and V units of different formats fill the same
// registers and the array never needs dynamic indexing.
struct ChunkRaw {
  uint32_t w[16];  // 9 dwords of a quantized block, the 16 of an f16 block
};

// Register holding dword i of a unit of format F.
template <int F>
__device__ constexpr int raw_slot(int i) { return F == MAB_KV_Q4 && i == 4 ? 8 : i; }

// WIDE: the other side (K or V) of the kernel uses 8-bit blocks; a 4-bit
// unit then takes the same three loads (the second a repeat of the first,
// unused) so that both sides' loads have one shape.
template <int F, bool WIDE = false>
__device__ inline void chunk_raw_load_al(ChunkRaw& r, const uint32_t* base) {
  if constexpr (F == MAB_KV_F16) {  // 64-byte blocks: always 16-byte aligned
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(base + 4 * i);
      r.w[4 * i] = x[0]; r.w[4 * i + 1] = x[1]; r.w[4 * i + 2] = x[2]; r.w[4 * i + 3] = x[3];
    }
  } else if constexpr (F == MAB_KV_Q8) {
    const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(base);
    const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(base + 4);
    r.w[0] = x0[0]; r.w[1] = x0[1]; r.w[2] = x0[2]; r.w[3] = x0[3];
    r.w[4] = x1[0]; r.w[5] = x1[1]; r.w[6] = x1[2]; r.w[7] = x1[3];
    r.w[8] = base[8];
  } else {
    const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(base);
    r.w[0] = x0[0]; r.w[1] = x0[1]; r.w[2] = x0[2]; r.w[3] = x0[3];
    if constexpr (WIDE) {
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(base);
      r.w[4] = x1[0]; r.w[5] = x1[1]; r.w[6] = x1[2]; r.w[7] = x1[3];
    }
    r.w[raw_slot<F>(4)] = base[4];
  }
}

template <int F, bool WIDE = false>
__device__ inline void chunk_raw_load(ChunkRaw& r, const uint8_t* blk) {
  const uintptr_t addr = reinterpret_cast<uintptr_t>(blk);
  chunk_raw_load_al<F, WIDE>(r, reinterpret_cast<const uint32_t*>(addr & ~(uintptr_t)3));
}

// Dword m of the unit's codes (codes 4m .. 4m+3, or nibbles 8m .. 8m+7) and
// the unit's fp16 scale bits.  The block starts at byte SH (0 or 2) of w, so
// its codes start at byte 2 or 4.
template <int F, int SH>
__device__ inline uint32_t raw_codes(const ChunkRaw& r, int m) {
  const uint32_t hi = r.w[raw_slot<F>(m + 1)];
  return SH ? hi : __builtin_amdgcn_alignbyte(hi, r.w[raw_slot<F>(m)], 2);
}
template <int SH>
__device__ inline uint32_t raw_scale(const ChunkRaw& r) { return SH ? r.w[0] >> 16 : r.w[0] & 0xFFFFu; }

// Writes unit (key, block b) of K (IS_V false) or V, in format F, into tile
// t.  A key past the range (its bytes come from a valid key) gets scale 0: K
// logits and V values of 0, never a stray NaN.  c = sm_scale*log2(e) is
// folded into the K scale.
template <int NB, int F, bool IS_V, int SH>
__device__ inline void chunk_unit_store(ChunkTile<NB>& t, const ChunkRaw& r, int key, int b, bool valid, float c) {
  using T = ChunkTile<NB>;
  half_t d;
  half8_t out[4];
  if constexpr (F == MAB_KV_F16) {  // the values themselves, scale 1
    d = (half_t)1.f;
    // a key past the range holds whatever the pool holds there (possibly
    // NaN): zero its values, as a scale of 0 does for the quantized formats
#pragma unroll
    for (int g8 = 0; g8 < 4; ++g8)
      out[g8] = valid ? __builtin_bit_cast(half8_t, u32x4_t{r.w[4 * g8], r.w[4 * g8 + 1], r.w[4 * g8 + 2],
                                                            r.w[4 * g8 + 3]})
                      : half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  } else {
    d = __builtin_bit_cast(half_t, (uint16_t)raw_scale<SH>(r));
#pragma unroll
    for (int g8 = 0; g8 < 4; ++g8) {
      if constexpr (F == MAB_KV_Q8) out[g8] = codes8_q8(raw_codes<F, SH>(r, 2 * g8), raw_codes<F, SH>(r, 2 * g8 + 1));
      else out[g8] = codes8_q4(raw_codes<F, SH>(r, g8));
    }
  }
  if (!valid) d = (half_t)0.f;
  half_t* row = (IS_V ? t.v : t.k) + key * T::kStride + 32 * b;
  if constexpr (IS_V) {
    const half8_t dv = half8_t{d, d, d, d, d, d, d, d};
#pragma unroll
    for (int g8 = 0; g8 < 4; ++g8) *reinterpret_cast<half8_t*>(row + 8 * g8) = out[g8] * dv;
  } else {
#pragma unroll
    for (int g8 = 0; g8 < 4; ++g8) *reinterpret_cast<half8_t*>(row + 8 * g8) = out[g8];
    t.kd[b * kStepKeys + key] = (float)d * c;
  }
}

__device__ inline half4_t lds_tr16(const half_t* p) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  const s4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4_t*)(const_cast<half_t*>(p)));
  return __builtin_bit_cast(half4_t, x);
}

// One wave's chunk state: two 16-row tiles of one query head.  Lane l serves
// row l%16 of each tile; the four lanes of a row (l/16) hold different keys of
// S^T and different dims of O^T.
template <int NB>
struct ChunkWave {
  half8_t q[2][NB];    // Q^T operand: row 16*rt + l%16, block b, slots 8*(l/16) + [0,8)
  float4_t o[2][2 * NB];  // O^T: tile rt, dim slots 16*dt + 4*(l/16) + [0,4)
  float4_t l[2];       // row sums of P, from an MFMA against ones (all four entries equal)
  float m[2];          // running (stale) max of the logits, in exp2 units (-inf: no key yet)
  int limit[2];        // last visible key of the lane's row (-1 past the rows)
};

template <int NB, int KF>
__device__ inline void chunk_wave_init(ChunkWave<NB>& cw, const half_t* q0, int hq, int nrows, int limit0,
                                       int lane) {
  const int n = lane & 15, j = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = 16 * rt + n;
    const bool ok = r < nrows;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      half8_t v = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
      if (ok) v = *reinterpret_cast<const half8_t*>(q0 + (int64_t)r * hq * (32 * NB) + 32 * b + 8 * j);
      cw.q[rt][b] = KF == MAB_KV_Q4 ? nibble_order(v) : v;
    }
#pragma unroll
    for (int t = 0; t < 2 * NB; ++t) cw.o[rt][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    cw.m[rt] = -INFINITY;
    cw.l[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
    cw.limit[rt] = ok ? limit0 + r : -1;
  }
}

// One 32-key step of a wave on tile t (keys kbase .. kbase+31, those at or
// past kend zeroed).  Logits are in exp2 units (the block scales in the tile
// already carry c = sm_scale*log2(e)) and relative to the row's running max m,
// so P = exp2(S).  `masked`: some key of the step lies past a row's limit or
// past kend.
template <int NB>
__device__ inline void chunk_step(ChunkWave<NB>& cw, const ChunkTile<NB>& t, int kbase, int kend, bool masked,
                                  int lane) {
  using T = ChunkTile<NB>;
  const int n = lane & 15, j = lane >> 4;
  float4_t s[2][2];  // [key tile][row tile]
  // the QK products at a raised issue priority: the matrix cores get fed while
  // the other wave of the SIMD is in its softmax or dequantization
  __builtin_amdgcn_s_setprio(2);
  // every product first (16 independent MFMAs), then the block scales: the
  // scale FMAs never wait on an MFMA issued just before them
  float4_t pb[2][NB][2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const half_t* kr = t.k + (16 * kt + n) * T::kStride + 8 * j;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const half8_t ka = *reinterpret_cast<const half8_t*>(kr + 32 * b);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        pb[kt][b][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, cw.q[rt][b], float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
  }
  // s = c * (Q K^T) - m in exp2 units: each logit's chain of block-scale FMAs
  // (scales already times c) starts from -m, the row's stale max (0 for a
  // row with no key yet), so P = exp2(s) needs no further arithmetic
  float base[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) base[rt] = cw.m[rt] == -INFINITY ? 0.f : -cw.m[rt];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    s[kt][0] = float4_t{base[0], base[0], base[0], base[0]};
    s[kt][1] = float4_t{base[1], base[1], base[1], base[1]};
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4_t kd = *reinterpret_cast<const float4_t*>(&t.kd[b * kStepKeys + 16 * kt + 4 * j]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kt][rt][i] = __builtin_fmaf(kd[i], pb[kt][b][rt][i], s[kt][rt][i]);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  if (__builtin_amdgcn_readfirstlane((int)masked)) {
    __builtin_amdgcn_sched_barrier(0);  // keeps the masking a taken-or-skipped branch
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kbase + 16 * kt + 4 * j + i;
          if (key > cw.limit[rt] || key >= kend) s[kt][rt][i] = -INFINITY;
        }
  }
  // Rescale only when a row's max grows by more than 2^kRescaleSlack (also
  // for a row's first visible keys): s is relative to the stale max, so the
  // test is s > slack.  A row's max passes only if one of its lanes' values
  // does: the lane-swap reductions and the rescale run only then (rarely after
  // the first steps), and shift that row's s to the new max.
  float lmx[2], thr[2];
  bool over = false;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    lmx[rt] = fmaxf(fmaxf(fmaxf(s[0][rt][0], s[0][rt][1]), fmaxf(s[0][rt][2], s[0][rt][3])),
                    fmaxf(fmaxf(s[1][rt][0], s[1][rt][1]), fmaxf(s[1][rt][2], s[1][rt][3])));
    thr[rt] = cw.m[rt] == -INFINITY ? -INFINITY : kRescaleSlack;
    over |= lmx[rt] > thr[rt];
  }
  if (__any(over)) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float mx = max_xor32(max_xor16(lmx[rt]));
      const bool grow = mx > thr[rt];
      if (__any(grow)) {
        const bool fresh = cw.m[rt] == -INFINITY;
        // 0 for a row's first keys (O and l are still 0); 1 for rows whose max stands
        const float alpha = grow ? (fresh ? 0.f : __builtin_amdgcn_exp2f(-mx)) : 1.f;
        const float shift = grow ? mx : 0.f;
#pragma unroll
        for (int dt = 0; dt < 2 * NB; ++dt) cw.o[rt][dt] *= alpha;
        cw.l[rt] *= alpha;
        if (grow) cw.m[rt] = (fresh ? 0.f : cw.m[rt]) + mx;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s[kt][rt] -= shift;
      }
    }
  }
  half8_t pf[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float p[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[4 * kt + i] = __builtin_amdgcn_exp2f(s[kt][rt][i]);  // <= 2^slack; masked 0
    pf[rt] = half8_t{(half_t)p[0], (half_t)p[1], (half_t)p[2], (half_t)p[3],
                     (half_t)p[4], (half_t)p[5], (half_t)p[6], (half_t)p[7]};
    // the row sums of the fp16 P that the PV products use, on the matrix cores
    const half8_t ones = half8_t{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    cw.l[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[rt], cw.l[rt], 0, 0, 0);
  }
  // V^T operand of dim slot 16*dt + n: keys 4j+[0,4) then 16+4j+[0,4), read by
  // two transpose reads in which lane n names row (key 4j+n/4 (+16), slots 16dt+4(n%4)+[0,4))
  const half_t* vr0 = t.v + (4 * j + (n >> 2)) * T::kStride + 4 * (n & 3);
  const half_t* vr1 = vr0 + 16 * T::kStride;
#pragma unroll
  for (int dt = 0; dt < 2 * NB; ++dt) {
    const half4_t a0 = lds_tr16(vr0 + 16 * dt);
    const half4_t a1 = lds_tr16(vr1 + 16 * dt);
    const half8_t va = half8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
      cw.o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pf[rt], cw.o[rt][dt], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Launch plan.  The grid holds the chunk work items first (one work-group per
// row tile and KV head), then the decode stream: the stages of every decode
// segment (one decode row and KV head) laid end to end, cut into equal
// contiguous ranges, one per decode worker (a wave; the decode work-groups
// hold 4 or 8 of them), so every wave streams the same number of bytes with
// no synchronisation.  A range that holds a whole segment writes its output;
// pieces of a longer segment write partials that combine_kernel merges in
// range order.
// ---------------------------------------------------------------------------

// Launch-order tables of the sequences.  Decode entry e (a one-row sequence):
// its Hkv segments of dec_stages(ctx) stages each start at dec_unit[e] +
// g*dec_stages(ctx).  Chunk entry c: work items [ch_item[c], ch_item[c+1]),
// ch_split[c] per tile.
// Small batches carry them in the kernel arguments; larger ones have
// plan_kernel write them to the workspace.
constexpr int kArgDec = 96;
constexpr int kArgChunk = 16;

struct ArgTabs {
  int dec_unit[kArgDec + 1], dec_seq[kArgDec], dec_r0[kArgDec], dec_ctx[kArgDec], dec_ntok[kArgDec];
  int ch_item[kArgChunk + 1], ch_seq[kArgChunk], ch_r0[kArgChunk], ch_qlen[kArgChunk], ch_prefix[kArgChunk];
  int ch_split[kArgChunk];
};

// Offsets (in ints) of the tables in the workspace.
struct WsTabs {
  int dec_unit, dec_seq, dec_r0, dec_ctx, dec_ntok, ch_item, ch_seq, ch_r0, ch_qlen, ch_prefix, ch_split, total;
};

__host__ __device__ inline WsTabs ws_tabs(int n_dec, int n_chunk) {
  WsTabs t;
  int o = 0;
  t.dec_unit = o; o += n_dec + 1;
  t.dec_seq = o; o += n_dec;
  t.dec_r0 = o; o += n_dec;
  t.dec_ctx = o; o += n_dec;
  t.dec_ntok = o; o += n_dec;
  t.ch_item = o; o += n_chunk + 1;
  t.ch_seq = o; o += n_chunk;
  t.ch_r0 = o; o += n_chunk;
  t.ch_qlen = o; o += n_chunk;
  t.ch_prefix = o; o += n_chunk;
  t.ch_split = o; o += n_chunk;
  t.total = o;
  return t;
}

struct AttnArgs {
  const half_t* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* q_start;
  const int32_t* prefix_len;
  const int32_t* block_table;
  float* out;
  float* o_part;           // decode partials [slot][G][D]
  float2* ml_part;         // [slot][G]
  float* ch_o;             // chunk partials [item][G][rows][D]
  float2* ch_ml;           // [item][G][rows]
  DirEntry* dir;
  int32_t* ws_tab;
  int num_seqs, max_pages;
  int hq, hkv, page_size;
  int n_dec, n_chunk;       // decode and chunk sequences
  int n_chunk_items;        // chunk work items (the first entries of the grid)
  int ch_target;            // work-group slots the chunk splits aim to fill
  int dec_units;            // units in the decode stream (stages, plus padding with dec_piece)
  int dec_piece;            // 0: equal ranges over the stream; else stages per piece (MAB_BATCH_INVARIANT)
  int dec_wide;             // verify sub-rows may take two slot groups (quantized pools)
  int dec_range;            // stages per decode worker (the last may have fewer)
  int dec_pmax;             // partial slots per decode worker
  int dec_slots;            // (row, head) slots of a decode partial: G, or T*G with verify rows
  int tabs_in_ws;           // tables in the workspace (1) or in `tabs` (0)
  float c;                  // sm_scale * log2(e)
  ArgTabs tabs;
  int num_pages;            // pages of each pool (page ids are checked against it in debug mode)
};

struct TabView {
  const int *dec_unit, *dec_seq, *dec_r0, *dec_ctx, *dec_ntok;
  const int *ch_item, *ch_seq, *ch_r0, *ch_qlen, *ch_prefix, *ch_split;
};

__device__ inline TabView tab_view(const AttnArgs& a) {
  TabView v;
  if (a.tabs_in_ws) {
    const WsTabs t = ws_tabs(a.n_dec, a.n_chunk);
    const int* b = a.ws_tab;
    v.dec_unit = b + t.dec_unit; v.dec_seq = b + t.dec_seq; v.dec_r0 = b + t.dec_r0; v.dec_ctx = b + t.dec_ctx;
    v.dec_ntok = b + t.dec_ntok;
    v.ch_item = b + t.ch_item; v.ch_seq = b + t.ch_seq; v.ch_r0 = b + t.ch_r0; v.ch_qlen = b + t.ch_qlen;
    v.ch_prefix = b + t.ch_prefix;
    v.ch_split = b + t.ch_split;
  } else {
    v.dec_unit = a.tabs.dec_unit; v.dec_seq = a.tabs.dec_seq; v.dec_r0 = a.tabs.dec_r0; v.dec_ctx = a.tabs.dec_ctx;
    v.dec_ntok = a.tabs.dec_ntok;
    v.ch_item = a.tabs.ch_item; v.ch_seq = a.tabs.ch_seq; v.ch_r0 = a.tabs.ch_r0; v.ch_qlen = a.tabs.ch_qlen;
    v.ch_prefix = a.tabs.ch_prefix;
    v.ch_split = a.tabs.ch_split;
  }
  return v;
}

// Index of the last entry e < n with base[e] <= x (base strictly increasing,
// base[0] <= x): every lane tests one entry per pass, so the search costs one
// round trip per 64 entries instead of a chain of dependent loads.
__device__ inline int wave_find(const int* base, int n, int x) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int e = e0 + lane;
    const bool le = e < n && base[e] <= x;
    cnt += __popcll(__ballot(le));
  }
  return cnt - 1;
}

template <int NB, int KF>
__device__ inline void dec_init(Group<NB>& gr, const half_t* qrow, int limit, int lane) {
  group_init(gr, qrow, limit, lane);
  if constexpr (KF == MAB_KV_Q4) {  // match the (0,2,4,6,1,3,5,7) order of 4-bit K codes
#pragma unroll
    for (int b = 0; b < NB; ++b) gr.q[b] = nibble_order(gr.q[b]);
  }
}

// One piece of a decode segment (ntok rows from row r0 of sequence s, the
// last of which sees ctx keys, KV head g, keys [kb, ke), kb a multiple of 32),
// streamed by one wave; slot n of the wave is row r0 + n/G, head g*G + n%G: 32-key stages, DEPTH
// stages ahead, with loads that bypass the caches' retention (every byte is
// read once), through the wave's own LDS stage buffer wbuf.  A whole segment
// writes the output, a piece its partial at `slot`.
template <int NB, int KF, int VF, int DEPTH, bool DBG>
__device__ inline void decode_piece(const AttnArgs& a, uint8_t* wbuf, int s, int r0, int ntok, int ctx, int g,
                                    int kb, int ke, bool whole, int64_t slot) {
  constexpr int D = 32 * NB;
  const int lane = threadIdx.x & 63;
  const int G = a.hq / a.hkv;
  const int n = lane & 15, j = lane >> 4;
  ItemCtx ic;
  ic.k_pool = a.k_pool;
  ic.v_pool = a.v_pool;
  ic.bt_row = a.block_table + (int64_t)s * a.max_pages;
  ic.hkv = a.hkv;
  ic.g = g;
  ic.page_size = a.page_size;
  const int nst = ceil_div(ke - kb, kStepKeys);
  // page ids of the piece's 16-key runs, 64 at a time (one per lane)
  auto page_window = [&](int win) {
    const int key = kb + 16 * (64 * win + lane);
    return key < ke ? checked_page(gload_i32(ic.bt_row + key / a.page_size), a.num_pages, DBG) : 0;
  };
  int my_page = page_window(0);
  const int tn = n / G, hn = n % G;  // this lane's slot: row r0 + tn, head g*G + hn
  const bool live = tn < ntok;
  const int64_t orow = (int64_t)(r0 + tn) * a.hq + g * G + hn;
  Group<NB> grs[1];
  Group<NB>& gr = grs[0];
  dec_init<NB, KF>(gr, live ? a.q + orow * D : nullptr, ctx - ntok + tn, lane);
  // a finite floor for the running max: a verify row's slot may see no key of
  // a piece that starts past its limit, and exp2(-inf - floor) is 0, not NaN
  gr.m = kDecodeMaxFloor;
  const int kvis = min(ke, ctx - ntok + 1);  // keys below this are visible to every live slot
  // DEPTH register sets: stage st is consumed from set st % DEPTH while the
  // next DEPTH-1 stages load into the others; its set is refilled with stage
  // st + DEPTH as soon as it is in LDS
  DecWave<NB, KF, VF> d[DEPTH];
  auto page_of_run = [&](int run) {  // wave-uniform; run is even on every window reload
    if (run > 0 && (run & 63) == 0) my_page = page_window(run >> 6);
    return __builtin_amdgcn_readlane(my_page, run & 63);
  };
  const bool one_page = a.page_size % kStepKeys == 0;  // every stage inside one page (kb % 32 == 0)
  auto issue = [&](DecWave<NB, KF, VF>& dw, int st) {
    const int run = 2 * st;
    const int p0 = page_of_run(run);
    if (one_page) dw.load_page(ic, kb + st * kStepKeys, p0, lane);
    else dw.load(ic, kb + st * kStepKeys, ke, p0, __builtin_amdgcn_readlane(my_page, (run + 1) & 63), lane);
  };
  auto consume = [&](DecWave<NB, KF, VF>& dw, int st) {
    const int kbase = kb + st * kStepKeys;
    dw.store(wbuf, lane);
    asm volatile("" ::: "memory");
    const bool big_v = dec_scales<NB, KF, VF>(wbuf, wbuf, lane, a.c, ke - kbase);
    if (st + DEPTH < nst) issue(dw, st + DEPTH);
    asm volatile("" ::: "memory");
    dec_compute<NB, KF, VF, 1>(grs, wbuf, wbuf, kbase, ke, kbase + kStepKeys > kvis, big_v, lane);
    asm volatile("" ::: "memory");
  };
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    if (i < nst) issue(d[i], i);
  for (int st = 0; st < nst; st += DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
      if (st + i < nst) consume(d[i], st + i);
  }
  float lsum = gr.l;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (!live) return;
  // remove the code bias: o -= bias * (sum of the block's weights)
  if constexpr (VBias<VF>::kBias != 0.f) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) gr.o[2 * b + t2] -= VBias<VF>::kBias * gr.vb[b][0];
  }
  const float inv = whole ? 1.f / lsum : 1.f;
  const int64_t pi = slot * a.dec_slots + n;
  float* dst = whole ? a.out + orow * D : a.o_part + pi * D;
  // lane (n, j) holds rows 4j + [0,4) of each block's two tiles, i.e. values
  // 8j + 2r + t2 (o[2b + t2][r]) of block b: eight consecutive dims of slot n
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float4_t* ob = &gr.o[2 * b];
    *reinterpret_cast<float4_t*>(dst + 32 * b + 8 * j) = float4_t{ob[0][0], ob[1][0], ob[0][1], ob[1][1]} * inv;
    *reinterpret_cast<float4_t*>(dst + 32 * b + 8 * j + 4) = float4_t{ob[0][2], ob[1][2], ob[0][3], ob[1][3]} * inv;
  }
  if (!whole && j == 0) a.ml_part[pi] = make_float2(gr.m, lsum);
}

// One piece of a wide verify sub-row (ntok rows, ntok*G > 16 slots): as
// decode_piece, with two groups of 16 slots that share every stage, slot
// 16k + n of group k being row r0 + (16k+n)/G, head g*G + (16k+n)%G.  The
// stage bytes go straight from memory into a ring of two LDS stage buffers
// (the registers hold the two groups' state instead): stage st + 1 is issued
// into the buffer that held stage st - 1 before the wave waits for stage st,
// so one stage is always in flight while another is computed on.  The
// compiler does not order LDS reads after these loads: the waits are
// explicit, and the LDS reads of a buffer are complete before it is refilled.
template <int NB, int KF, int VF, bool DBG>
__device__ inline void decode_piece_wide(const AttnArgs& a, uint8_t* wbuf, int s, int r0, int ntok, int ctx, int g,
                                         int kb, int ke, bool whole, int64_t slot) {
  using L = DecLayout<NB, KF, VF>;
  static_assert(L::kWideOk, "quantized pools only");
  // every argument is the same across the wave: say so, so that the stage
  // loop and the page walk run on the scalar unit
  s = __builtin_amdgcn_readfirstlane(s);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  ntok = __builtin_amdgcn_readfirstlane(ntok);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  g = __builtin_amdgcn_readfirstlane(g);
  kb = __builtin_amdgcn_readfirstlane(kb);
  ke = __builtin_amdgcn_readfirstlane(ke);
  constexpr int D = 32 * NB;
  const int lane = threadIdx.x & 63;
  const int G = a.hq / a.hkv;
  const int n = lane & 15, j = lane >> 4;
  const int32_t* bt_row = a.block_table + (int64_t)s * a.max_pages;
  const int nst = ceil_div(ke - kb, kStepKeys);
  // page ids of the piece's 16-key runs, 64 at a time (one per lane)
  auto page_window = [&](int win) {
    const int key = kb + 16 * (64 * win + lane);
    return key < ke ? checked_page(gload_i32(bt_row + key / a.page_size), a.num_pages, DBG) : 0;
  };
  int my_page = page_window(0);
  Group<NB> gr[2];
  bool live[2];
  int64_t orow[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int tn = (16 * k + n) / G, hn = (16 * k + n) % G;
    live[k] = tn < ntok;
    orow[k] = (int64_t)(r0 + tn) * a.hq + g * G + hn;
    dec_init<NB, KF>(gr[k], live[k] ? a.q + orow[k] * D : nullptr, ctx - ntok + tn, lane);
    gr[k].m = kDecodeMaxFloor;  // finite: a slot may see no key of the piece
#pragma unroll
    for (int b = 0; b < NB; ++b) gr[k].vs[b] = 0.f;
  }
  const int kvis = min(ke, ctx - ntok + 1);  // keys below this are visible to every live slot
  auto page_of_run = [&](int run) {
    if (run > 0 && (run & 63) == 0) {
      my_page = page_window(run >> 6);
      // wait here, on the rare path: a wait at the read below would sit on
      // every stage and hold the next stage's issue back for this one
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    return __builtin_amdgcn_readlane(my_page, run & 63);
  };
  // the ring: stage buffer 0 at the start of the wave area, 1 after the scales
  auto stage_buf = [&](int st) { return (st & 1) ? wbuf + L::kWaveBytes : wbuf; };
  auto issue = [&](int st) {
    const int key0 = kb + st * kStepKeys, key1 = key0 + 16;
    const int p0 = page_of_run(2 * st);
    const int p1 = __builtin_amdgcn_readlane(my_page, (2 * st + 1) & 63);  // same window: 2*st is even
    const int64_t tok0 = ((int64_t)p0 * a.hkv + g) * a.page_size + key0 % a.page_size;
    const int64_t tok1 = ((int64_t)p1 * a.hkv + g) * a.page_size + key1 % a.page_size;
    dec_stage_to_lds<NB, KF, VF>(stage_buf(st), a.k_pool + tok0 * L::kRecK,
                                 a.k_pool + tok1 * L::kRecK, a.v_pool + tok0 * L::kRecV, a.v_pool + tok1 * L::kRecV,
                                 key1 < ke, lane);
  };
  issue(0);
  for (int st = 0; st < nst; ++st) {
    const int kbase = kb + st * kStepKeys;
    if (st + 1 < nst) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage st - 1's reads of the buffer are done
      issue(st + 1);
      wait_vmcnt<L::run_load_issues()>();  // all but stage st + 1's loads have landed
    } else {
      wait_vmcnt<0>();
    }
    const uint8_t* raw = stage_buf(st);
    const bool big_v = dec_scales<NB, KF, VF>(raw, wbuf, lane, a.c, ke - kbase);
    dec_compute<NB, KF, VF, 2>(gr, raw, wbuf, kbase, ke, kbase + kStepKeys > kvis, big_v, lane);
    asm volatile("" ::: "memory");
  }
  float lsum[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    lsum[k] = gr[k].l;
    lsum[k] += __shfl_xor(lsum[k], 16);
    lsum[k] += __shfl_xor(lsum[k], 32);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      gr[k].vs[b] += __shfl_xor(gr[k].vs[b], 16);
      gr[k].vs[b] += __shfl_xor(gr[k].vs[b], 32);
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (!live[k]) continue;
    if constexpr (VBias<VF>::kBias != 0.f) {  // remove the code bias
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) gr[k].o[2 * b + t2] -= VBias<VF>::kBias * gr[k].vs[b];
    }
    const float inv = whole ? 1.f / lsum[k] : 1.f;
    const int64_t pi = slot * a.dec_slots + 16 * k + n;
    float* dst = whole ? a.out + orow[k] * D : a.o_part + pi * D;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4_t* ob = &gr[k].o[2 * b];
      *reinterpret_cast<float4_t*>(dst + 32 * b + 8 * j) = float4_t{ob[0][0], ob[1][0], ob[0][1], ob[1][1]} * inv;
      *reinterpret_cast<float4_t*>(dst + 32 * b + 8 * j + 4) =
          float4_t{ob[0][2], ob[1][2], ob[0][3], ob[1][3]} * inv;
    }
    if (!whole && j == 0) a.ml_part[pi] = make_float2(gr[k].m, lsum[k]);
  }
}

// Decode worker w (one wave): stages [w*R, min((w+1)*R, units)) of the decode
// stream, one piece per segment it touches.  The worker that runs a segment's
// first stage records where the segment's results went.
template <int NB, int KF, int VF, int DEPTH, bool DBG, bool WIDE>
__device__ inline void decode_worker(const AttnArgs& a, uint8_t* wbuf, int w) {
  const int x0 = w * a.dec_range, x1 = min(x0 + a.dec_range, a.dec_units);
  if (x0 >= x1) return;
  const TabView tv = tab_view(a);
  const int G = a.hq / a.hkv;
  int e = wave_find(tv.dec_unit, a.n_dec, x0);
  int x = x0, k = 0;
  while (x < x1) {
    const int ctx = tv.dec_ctx[e], ub = tv.dec_unit[e], ntok = tv.dec_ntok[e];
    const int nst = dec_units_of(ctx, a.dec_piece);   // the segment's units in the stream
    const int g = (x - ub) / nst;
    const int seg_lo = ub + g * nst, seg_hi = seg_lo + nst;
    const int work_hi = seg_lo + dec_stages(ctx);     // units past it are padding
    const int p_hi = min(x1, seg_hi);
    if (x < work_hi) {
      const int r0 = tv.dec_r0[e];
      const bool first = x == seg_lo, whole = first && p_hi >= work_hi;
      const int64_t slot = (int64_t)w * a.dec_pmax + k;
      const int kb = (x - seg_lo) * kStepKeys, ke = min(ctx, (p_hi - seg_lo) * kStepKeys);
      bool wide = false;  // more than 16 slots: two slot groups
      if constexpr (WIDE) {
        wide = ntok * G > 16;
        if (wide) decode_piece_wide<NB, KF, VF, DBG>(a, wbuf, tv.dec_seq[e], r0, ntok, ctx, g, kb, ke, whole, slot);
      }
      if (!wide) decode_piece<NB, KF, VF, DEPTH, DBG>(a, wbuf, tv.dec_seq[e], r0, ntok, ctx, g, kb, ke, whole, slot);
      if (first && (threadIdx.x & 63) == 0) {
        DirEntry d;
        d.slot = (int)slot;
        d.wg = w;
        d.n = whole ? 1 : (work_hi - 1) / a.dec_range - w + 1;
        d.rh0 = r0 * a.hq + g * G;
        a.dir[e * a.hkv + g] = d;
      }
      ++k;
    }
    x = p_hi;
    if (x == seg_hi && g + 1 == a.hkv) ++e;
  }
}

// Chunk work item: row tile qt (R rows) of a chunk sequence, KV head g, head
// group hp (H heads), keys [kb, ke) of the rows' visible range.  Wave (hh, rg)
// serves query head hp*H + hh of the group and rows 32*rg .. 32*rg+31 of the
// tile.  pslot < 0: the item covers every key of its rows and writes the
// output; otherwise its partial goes to slot pslot.  DBG: check page ids
// (debug mode; a separate instantiation keeps the checks out of the normal
// step loop).
template <int NB, int KF, int VF, bool DBG, bool UNIFORM>
__device__ inline void chunk_item(const AttnArgs& a, uint8_t* smem, const ItemCtx& ic, int r0, int q_len, int prefix,
                                  int g, int hp, int qt, int kb, int ke, int64_t pslot) {
  // every argument is the same across the work-group; say so, so that the
  // step loop and the page walk run on the scalar unit
  r0 = __builtin_amdgcn_readfirstlane(r0);
  q_len = __builtin_amdgcn_readfirstlane(q_len);
  prefix = __builtin_amdgcn_readfirstlane(prefix);
  g = __builtin_amdgcn_readfirstlane(g);
  hp = __builtin_amdgcn_readfirstlane(hp);
  qt = __builtin_amdgcn_readfirstlane(qt);
  kb = __builtin_amdgcn_readfirstlane(kb);
  ke = __builtin_amdgcn_readfirstlane(ke);
  constexpr int D = 32 * NB;
  constexpr int kUnits = 2 * kStepKeys * NB;  // dequant units of a step: (key, block) of K, then of V
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.hq / a.hkv, H = chunk_heads(G), R = chunk_rows(G);
  const int hh = wave % H, rg = wave / H, hl = hp * H + hh;
  ChunkTile<NB>* tiles = reinterpret_cast<ChunkTile<NB>*>(smem);

  const int row0 = qt * R + 32 * rg;  // the wave's first row within the chunk
  const int nrows = max(0, min(32, q_len - row0));
  ChunkWave<NB> cw;
  chunk_wave_init<NB, KF>(cw, a.q + ((int64_t)(r0 + row0) * a.hq + g * G + hl) * D, a.hq, nrows, prefix + row0,
                          lane);
  const int nst = ceil_div(ke - kb, kStepKeys);
  // Q is in registers before the step loop starts: the loads still pending
  // inside the loop are then only the step prefetches, and no product of the
  // loop waits for them
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // This thread's dequant unit: key tid%32 of one block of K or V.  Each wave
  // holds two units whose blocks have the same parity, hence the same byte
  // alignment in memory (records are a multiple of 4 bytes, blocks 34 or 18):
  // head_dim 128: waves 0,1 K blocks {0,2},{1,3}, waves 2,3 V; head_dim 64:
  // wave w K block w (lanes 0-31) and V block w (lanes 32-63).  The other
  // waves only compute (waves w and w+4 share a SIMD).
  const int half = (tid >> 5) & 1;
  const bool has_unit = wave < kUnits / 64;  // wave-uniform: the page walk stays scalar
  const bool u_is_v = NB == 4 ? wave >= 2 : half != 0;
  const int u_b = NB == 4 ? (wave & 1) + 2 * half : wave;
  const int u_key = tid & 31;
  const int ps = a.page_size;
  const uint8_t* pool = u_is_v ? ic.v_pool : ic.k_pool;
  const int rec = NB * (u_is_v ? Fmt<VF>::kBytes : Fmt<KF>::kBytes);
  const int boff = u_b * (u_is_v ? Fmt<VF>::kBytes : Fmt<KF>::kBytes);
  // byte offset of the unit's block in its dword (the same for every lane of a
  // wave: records are a multiple of 4 bytes, pools 16-byte aligned)
  const int sh = __builtin_amdgcn_readfirstlane(boff & 3);
  ChunkRaw raw_a, raw_b;  // the loads of two steps in flight: even steps in raw_a, odd ones in raw_b
  constexpr bool kWide = KF == MAB_KV_Q8 || VF == MAB_KV_Q8;
  auto dequant = [&](int st, const ChunkRaw& raw) {
    const bool valid = kb + st * kStepKeys + u_key < ke;
    ChunkTile<NB>& t = tiles[st & 1];
    if (u_is_v) {
      if (sh) chunk_unit_store<NB, VF, true, 2>(t, raw, u_key, u_b, valid, a.c);
      else chunk_unit_store<NB, VF, true, 0>(t, raw, u_key, u_b, valid, a.c);
    } else {
      if (sh) chunk_unit_store<NB, KF, false, 2>(t, raw, u_key, u_b, valid, a.c);
      else chunk_unit_store<NB, KF, false, 0>(t, raw, u_key, u_b, valid, a.c);
    }
  };
  // The loads of a step.  Page sizes that are a multiple of 32 keep every step
  // (which starts at a multiple of 32) inside one page: a wave-uniform page
  // walk (scalar page ids, the next page's id fetched a page ahead) and a
  // fixed per-lane offset.  Lanes past the range read bytes of the same page
  // and are zeroed by their scale.  Other page sizes take a per-lane walk.
  // (a separate instantiation per walk: a load pending on one walk's path
  // must not make the other wait for its own prefetches)
  constexpr bool uniform = UNIFORM;
  const uint32_t lane_off = (uint32_t)(u_key * rec + (boff & ~3));
  int u_q = kb / ps, u_r = kb % ps;  // page index and slot of the next step to load
  const int q_last = (ke - 1) / ps;
  // the block table is read-only during the call: scalar loads
  const __attribute__((address_space(4))) int32_t* bt_const =
      (const __attribute__((address_space(4))) int32_t*)(wave_uniform(ic.bt_row));
  int u_pg = 0, u_pg_next = 0, bad_page = 0;
  auto issue_uniform = [&](ChunkRaw& raw) {
    const uint8_t* base = pool + (((int64_t)u_pg * ic.hkv + g) * ps + u_r) * rec;
    if (u_is_v) chunk_raw_load_al<VF, kWide>(raw, reinterpret_cast<const uint32_t*>(base + lane_off));
    else chunk_raw_load_al<KF, kWide>(raw, reinterpret_cast<const uint32_t*>(base + lane_off));
    u_r += kStepKeys;
    if (u_r == ps) {
      u_r = 0;
      ++u_q;
      u_pg = u_pg_next;
      u_pg_next = u_q < q_last ? clamp_page(bt_const[u_q + 1], a.num_pages, DBG, bad_page) : 0;
    }
  };
  // per-lane walk: position of a step's first key (page index q, slot r),
  // advanced 32 keys at a time without dividing; a lane past the range reads
  // the step's first key
  struct Pos { int q, r; };
  auto advance = [&](Pos p) {
    p.r += kStepKeys;
    while (p.r >= ps) { p.r -= ps; ++p.q; }
    return p;
  };
  auto lane_page_slot = [&](Pos p, int st, int& pidx, int& slot) {
    const int t = kb + st * kStepKeys + u_key < ke ? p.r + u_key : p.r;
    const int c = (t >= ps) + (t >= 2 * ps);
    pidx = p.q + c;
    slot = t - c * ps;
  };
  int raw_slot = 0;
  auto issue_lane = [&](ChunkRaw& raw, int page) {  // the unit's own block only: the read never leaves the key's record
    const int64_t tok = ((int64_t)page * ic.hkv + g) * ps + raw_slot;
    if (u_is_v) chunk_raw_load<VF, kWide>(raw, pool + tok * rec + boff);
    else chunk_raw_load<KF, kWide>(raw, pool + tok * rec + boff);
  };
  // pipeline: the tile of step st+1 is filled from registers during step st,
  // whose loads were issued during step st-2 (per-lane walk: with page ids
  // fetched one issue earlier); two register sets hold the loads in flight
  Pos p_page = {kb / ps, kb % ps};  // step of the next page-id fetch
  int pidx, next_slot = 0, pg_next = 0;
  auto fetch_page = [&](int st) {
    lane_page_slot(p_page, st, pidx, next_slot);
    pg_next = clamp_page(ic.bt_row[pidx], a.num_pages, DBG, bad_page);
    p_page = advance(p_page);
  };
  auto issue = [&](int st, ChunkRaw& raw) {  // loads of step st (issued in step order)
    if constexpr (uniform) {
      issue_uniform(raw);
    } else {
      raw_slot = next_slot;
      issue_lane(raw, pg_next);
      if (st + 1 < nst) fetch_page(st + 1);
    }
  };
  if (has_unit && nst > 0) {
    if constexpr (uniform) {
      u_pg = clamp_page(bt_const[u_q], a.num_pages, DBG, bad_page);
      u_pg_next = u_q < q_last ? clamp_page(bt_const[u_q + 1], a.num_pages, DBG, bad_page) : 0;
    } else {
      fetch_page(0);
    }
    issue(0, raw_a);
    if (nst > 1) issue(1, raw_b);
    dequant(0, raw_a);
    if (nst > 2) issue(2, raw_a);
  }
  __syncthreads();
  // step st: the tile of step st+1 is filled from the set holding it (raw_b
  // for even st), whose loads were issued two steps earlier, and the set is
  // reloaded with step st+3
  auto body = [&](int st, ChunkRaw& raw) {
    const int kbase = kb + st * kStepKeys;
    if (has_unit && st + 1 < nst) {
      dequant(st + 1, raw);
      if (st + 3 < nst) issue(st + 3, raw);
    }
    // every wave computes (one past the last row on zero queries, written nowhere)
    const bool masked = kbase + kStepKeys - 1 > prefix + row0 || kbase + kStepKeys > ke;
    chunk_step<NB>(cw, tiles[st & 1], kbase, ke, masked, lane);
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 2) {
    body(st, raw_b);
    if (st + 1 < nst) body(st + 1, raw_a);
  }
  report_bad_page(bad_page);
  if (nrows == 0) return;
  const int n = lane & 15, j = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float ltot = cw.l[rt][0];
    const int r = 16 * rt + n;
    if (r >= nrows) continue;
    const int row_in_tile = 32 * rg + r;
    float* dst;
    float inv = 1.f;
    if (pslot < 0) {
      dst = a.out + ((int64_t)(r0 + row0 + r) * a.hq + g * G + hl) * D;
      inv = 1.f / ltot;
    } else {
      const int64_t pi = (pslot * H + hh) * R + row_in_tile;
      dst = a.ch_o + pi * D;
      if (j == 0) a.ch_ml[pi] = make_float2(cw.m[rt], ltot);
    }
#pragma unroll
    for (int dt = 0; dt < 2 * NB; ++dt) {
      const float4_t o = cw.o[rt][dt] * inv;
      if constexpr (VF != MAB_KV_Q4) {  // natural value order
        *reinterpret_cast<float4_t*>(dst + 16 * dt + 4 * j) = o;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[value_of_slot<VF>(16 * dt + 4 * j + i)] = o[i];
      }
    }
  }
}

// Chunk work item `item` of chunk entry c: tile (local / F) = row tile qt, KV
// head g and head group hp, key split (local % F) of F = ch_split[c].  The visible keys of
// the tile's rows, [0, prefix + last row + 1), are cut into F ranges of whole
// steps.
template <int NB, int KF, int VF, bool DBG>
__device__ inline void chunk_work(const AttnArgs& a, uint8_t* smem, int item) {
  const TabView tv = tab_view(a);
  const int c = wave_find(tv.ch_item, a.n_chunk, item);
  const int local = item - tv.ch_item[c], F = tv.ch_split[c];
  const int r0 = tv.ch_r0[c], q_len = tv.ch_qlen[c], prefix = tv.ch_prefix[c];
  const int G = a.hq / a.hkv, H = chunk_heads(G), R = chunk_rows(G);
  const int n_qt = ceil_div(q_len, R), n_hp = G / H;
  const int tile = local / F, j = local % F;
  const ChunkTileCoord tc = chunk_tile_coord(tile, n_qt, n_hp, a.hkv);
  const int qt = tc.qt, hp = tc.hp, g = tc.g;
  ItemCtx ic;
  ic.k_pool = a.k_pool;
  ic.v_pool = a.v_pool;
  ic.bt_row = a.block_table + (int64_t)tv.ch_seq[c] * a.max_pages;
  ic.hkv = a.hkv;
  ic.g = g;
  ic.page_size = a.page_size;
  const int tile_end = prefix + min(q_len, (qt + 1) * R);  // keys past the tile's last row are never seen
  if (F == 1) {
    if (a.page_size % kStepKeys == 0) chunk_item<NB, KF, VF, DBG, true>(a, smem, ic, r0, q_len, prefix, g, hp, qt, 0, tile_end, -1);
    else chunk_item<NB, KF, VF, DBG, false>(a, smem, ic, r0, q_len, prefix, g, hp, qt, 0, tile_end, -1);
    return;
  }
  const int len = ceil_div(ceil_div(tile_end, F), kStepKeys) * kStepKeys;
  const int kb = min(j * len, tile_end), ke = min(kb + len, tile_end);
  if (kb < ke) {
    if (a.page_size % kStepKeys == 0) chunk_item<NB, KF, VF, DBG, true>(a, smem, ic, r0, q_len, prefix, g, hp, qt, kb, ke, item);
    else chunk_item<NB, KF, VF, DBG, false>(a, smem, ic, r0, q_len, prefix, g, hp, qt, kb, ke, item);
  } else {  // an empty split: a neutral partial (no keys) for every row of the tile
    const int64_t base = (int64_t)item * H * R;
    for (int u = threadIdx.x; u < H * R; u += blockDim.x) a.ch_ml[base + u] = make_float2(-INFINITY, 0.f);
  }
}

template <int NB, int KF, int VF, bool HAS_CHUNK, bool DBG, bool WIDE>
__device__ inline void attention_body(const AttnArgs& a, uint8_t* smem) {
  const int b = blockIdx.x;
  if constexpr (HAS_CHUNK) {
    if (b < a.n_chunk_items) {
      chunk_work<NB, KF, VF, DBG>(a, smem, b);
      return;
    }
  }
  constexpr int nw = HAS_CHUNK ? kMixedWaves : kDecodeWaves;
  const int wave = threadIdx.x >> 6;
  using L = DecLayout<NB, KF, VF>;
  decode_worker<NB, KF, VF, kDecodeDepth, DBG, WIDE>(a, smem + wave * (WIDE ? L::kWideBytes : L::kWaveBytes),
                                         (b - a.n_chunk_items) * nw + wave);
}

// One stage buffer per wave, two with wide verify pieces (WIDE).
template <int NB, int KF, int VF, bool WIDE>
constexpr int decode_smem_bytes(int waves) {
  return waves * (WIDE ? DecLayout<NB, KF, VF>::kWideBytes : DecLayout<NB, KF, VF>::kWaveBytes);
}

template <int NB, int KF, int VF, bool WIDE>
constexpr int mixed_smem_bytes() {
  const int dec = decode_smem_bytes<NB, KF, VF, WIDE>(kMixedWaves);
  const int chunk = 2 * (int)sizeof(ChunkTile<NB>);
  return dec > chunk ? dec : chunk;
}

// The decode path comes in two builds: without and with the wide verify
// pieces.  A batch whose decode rows all fit one slot group takes the first,
// whose registers and waits the second's code would otherwise disturb.

// Batches with a chunk: chunk tiles and decode stream ranges in one launch of
// kMixedWaves-wave work-groups, two waves per SIMD (one work-group per
// compute unit).
template <int NB, int KF, int VF, bool DBG, bool WIDE>
__global__ void __launch_bounds__(64 * kMixedWaves) __attribute__((amdgpu_waves_per_eu(2, 8)))
mixed_attention_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[mixed_smem_bytes<NB, KF, VF, WIDE>()];
  attention_body<NB, KF, VF, true, DBG, WIDE>(a, smem);
}

// Decode-only batches: kDecodeWaves waves per work-group, two per SIMD (room
// for two stages in flight per wave).
template <int NB, int KF, int VF, bool DBG, bool WIDE>
__global__ void __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(2, 8)))
decode_attention_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[decode_smem_bytes<NB, KF, VF, WIDE>(kDecodeWaves)];
  attention_body<NB, KF, VF, false, DBG, WIDE>(a, smem);
}

// Merges the pieces of decode segments that span several decode workers.
// One work-group per (segment, slot, 1/SPLIT of the dims), slot n being row
// n/G of the segment's sub-row and query head n%G of the group: thread (phase
// ph, dims 4q..4q+3) folds pieces ph, ph+P, ph+2P, ... into a running
// (m, l, o) with up to sixteen 16-byte loads in flight, then the P phases are
// folded pairwise in a fixed tree.  P = 8 over all dims, or, when some
// segment has more than kCombineWidePieces pieces (few long rows), P = 32
// over 32 dims per work-group.  The order depends only on the piece count
// and P: deterministic.
constexpr int kCombineUnroll = 16;
constexpr int kCombineWidePieces = 128;

__device__ inline void lse_fold(float& m, float& l, float4_t& o, float m2, float l2, float4_t o2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  const float a1 = __builtin_amdgcn_exp2f(m - mn), a2 = __builtin_amdgcn_exp2f(m2 - mn);
  l = l * a1 + l2 * a2;
  o = o * a1 + o2 * a2;
  m = mn;
}

template <int P, int NB, int SPLIT>
__global__ void __launch_bounds__(8 * NB / SPLIT * P)
combine_kernel(AttnArgs a) {
  constexpr int DQ = 8 * NB / SPLIT, D = 32 * NB;  // threads per phase (four dims each), head_dim
  __shared__ float4_t red_o[DQ * P];
  __shared__ float2 red_ml[DQ * P];
  const int G = a.hq / a.hkv, S = a.dec_slots;
  const int wg = blockIdx.x / SPLIT, part = blockIdx.x % SPLIT;
  const int seg = wg / S, hl = wg % S;
  const int q4 = part * DQ + threadIdx.x % DQ, ph = threadIdx.x / DQ;
  const DirEntry d = a.dir[seg];
  const int ntok = tab_view(a).dec_ntok[seg / a.hkv];
  if (d.n <= 1 || hl >= ntok * G) return;  // one piece, or a slot past the sub-row's rows
  auto slot = [&](int p) -> int64_t { return p == 0 ? d.slot : (int64_t)(d.wg + p) * a.dec_pmax; };
  float m = -INFINITY, l = 0.f;
  float4_t o = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int p0 = ph; p0 < d.n; p0 += P * kCombineUnroll) {
    float2 ml[kCombineUnroll];
    float4_t ov[kCombineUnroll];
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      const int p = p0 + P * u;
      ml[u] = make_float2(-INFINITY, 0.f);
      ov[u] = float4_t{0.f, 0.f, 0.f, 0.f};
      if (p < d.n) {
        const int64_t pi = slot(p) * S + hl;
        ml[u] = a.ml_part[pi];
        ov[u] = *reinterpret_cast<const float4_t*>(a.o_part + pi * D + 4 * q4);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) lse_fold(m, l, o, ml[u].x, ml[u].y, ov[u]);
  }
  // fixed pairwise tree over the phases: phase ph takes phase ph + half
  for (int half = P / 2; half >= 1; half >>= 1) {
    red_o[threadIdx.x] = o;
    red_ml[threadIdx.x] = make_float2(m, l);
    __syncthreads();
    if (ph < half) {
      const int t = threadIdx.x + DQ * half;
      const float2 ml2 = red_ml[t];
      lse_fold(m, l, o, ml2.x, ml2.y, red_o[t]);
    }
    __syncthreads();
  }
  if (ph == 0)
    *reinterpret_cast<float4_t*>(a.out + ((int64_t)d.rh0 + (int64_t)(hl / G) * a.hq + hl % G) * D + 4 * q4) =
        o / l;
}

// Merges the key splits of chunk tiles cut into more than one split.  A tile
// holds H*R = 32*kMixedWaves rows (all its heads); its F split items each
// own kChunkCombineGroups work-groups, and work-group q of split j merges
// the tile's rows [(j*kChunkCombineGroups + q)*per, ...+per), per =
// ceil(H*R / (F*kChunkCombineGroups)), so no work-group is idle: thread
// (row, 4 dims) takes the global max of the splits' maxima, then sums the
// weighted partials in split order, with every split's loads in flight
// together.  Deterministic.
constexpr int kChunkCombineThreads = 256;
constexpr int kChunkCombineGroups = 8;  // work-groups per split item

__global__ void __launch_bounds__(kChunkCombineThreads)
chunk_combine_kernel(AttnArgs a, int head_dim) {
  const TabView tv = tab_view(a);
  const int item = blockIdx.x / kChunkCombineGroups, q = blockIdx.x % kChunkCombineGroups;
  const int c = wave_find(tv.ch_item, a.n_chunk, item);
  const int local = item - tv.ch_item[c], F = tv.ch_split[c];
  if (F == 1) return;
  const int j = local % F, first = item - j;  // the tile's split 0
  const int r0 = tv.ch_r0[c], q_len = tv.ch_qlen[c];
  const int G = a.hq / a.hkv, H = chunk_heads(G), R = chunk_rows(G);
  const int n_qt = ceil_div(q_len, R), n_hp = G / H;
  const ChunkTileCoord tc = chunk_tile_coord(local / F, n_qt, n_hp, a.hkv);
  const int qt = tc.qt, hp = tc.hp, g = tc.g;
  const int tpr = head_dim / 4;                           // threads per row
  const int rpp = kChunkCombineThreads / tpr;             // rows per pass
  const int per = ceil_div(H * R, F * kChunkCombineGroups);
  const int lo = (j * kChunkCombineGroups + q) * per, hi = min(H * R, lo + per);
  const int dd = 4 * (threadIdx.x % tpr);
  for (int rt = lo + threadIdx.x / tpr; rt < hi; rt += rpp) {  // row of the tile, head-major
    const int hh = rt / R, rr = rt % R;
    const int i = qt * R + rr;
    if (i >= q_len) continue;
    float2 ml[kMaxChunkSplit];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kMaxChunkSplit; ++jj) {
      ml[jj] = make_float2(-INFINITY, 0.f);
      if (jj < F) ml[jj] = a.ch_ml[((int64_t)(first + jj) * H + hh) * R + rr];
      mx = fmaxf(mx, ml[jj].x);
    }
    float l = 0.f;
    float4_t o = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < kMaxChunkSplit; ++jj) {
      if (jj < F && ml[jj].y > 0.f) {  // an empty split (no keys) has l = 0 and unwritten o
        const float w = __builtin_amdgcn_exp2f(ml[jj].x - mx);
        const int64_t pi = ((int64_t)(first + jj) * H + hh) * R + rr;
        l += w * ml[jj].y;
        o += w * *reinterpret_cast<const float4_t*>(a.ch_o + pi * head_dim + dd);
      }
    }
    *reinterpret_cast<float4_t*>(a.out + ((int64_t)(r0 + i) * a.hq + g * G + hp * H + hh) * head_dim + dd) = o / l;
  }
}

// Writes the launch-order tables to the workspace for batches too large for
// the kernel arguments: one work-group, each thread classifies a contiguous
// range of sequences, ranges are placed by a work-group exclusive scan.
constexpr int kPlanThreads = 1024;

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(AttnArgs a) {
  __shared__ int scan[4][kPlanThreads];
  const int tid = threadIdx.x;
  const int G = a.hq / a.hkv;
  const int per = ceil_div(a.num_seqs, kPlanThreads);
  const int s0 = min(a.num_seqs, tid * per), s1 = min(a.num_seqs, s0 + per);
  int v[4] = {0, 0, 0, 0};  // decode entries, decode units, chunk entries, chunk items
  for (int s = s0; s < s1; ++s) {
    const int q_len = a.q_start[s + 1] - a.q_start[s], ctx = a.prefix_len[s] + q_len;
    if (is_chunk(q_len)) {
      const int tiles = chunk_tiles(q_len, a.hkv, G);
      v[2] += 1;
      v[3] += tiles * chunk_split(tiles, a.ch_target);
    } else {
      for (int i = 0, T = dec_tokens(q_len, G, a.dec_wide); i < dec_subrows(q_len, G, a.dec_wide); ++i) {
        v[0] += 1;
        v[1] += a.hkv * dec_units_of(ctx - q_len + min(q_len, (i + 1) * T), a.dec_piece);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) scan[k][tid] = v[k];
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {  // inclusive Hillis-Steele scan
    int t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = tid >= off ? scan[k][tid - off] : 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) scan[k][tid] += t[k];
    __syncthreads();
  }
  int base[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) base[k] = scan[k][tid] - v[k];
  const WsTabs t = ws_tabs(a.n_dec, a.n_chunk);
  int* w = a.ws_tab;
  for (int s = s0; s < s1; ++s) {
    const int r0 = a.q_start[s], q_len = a.q_start[s + 1] - r0, prefix = a.prefix_len[s];
    if (is_chunk(q_len)) {
      const int c = base[2]++;
      w[t.ch_item + c] = base[3];
      w[t.ch_seq + c] = s;
      w[t.ch_r0 + c] = r0;
      w[t.ch_qlen + c] = q_len;
      w[t.ch_prefix + c] = prefix;
      const int tiles = chunk_tiles(q_len, a.hkv, G), f = chunk_split(tiles, a.ch_target);
      w[t.ch_split + c] = f;
      base[3] += tiles * f;
    } else {
      for (int i = 0, T = dec_tokens(q_len, G, a.dec_wide); i < dec_subrows(q_len, G, a.dec_wide); ++i) {
        const int e = base[0]++, t1 = min(q_len, (i + 1) * T);
        w[t.dec_unit + e] = base[1];
        w[t.dec_seq + e] = s;
        w[t.dec_r0 + e] = r0 + i * T;
        w[t.dec_ctx + e] = prefix + t1;
        w[t.dec_ntok + e] = t1 - i * T;
        base[1] += a.hkv * dec_units_of(prefix + t1, a.dec_piece);
      }
    }
  }
  if (tid == kPlanThreads - 1) {
    w[t.dec_unit + a.n_dec] = scan[1][tid];
    w[t.ch_item + a.n_chunk] = scan[3][tid];
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

bool fmt_ok(int32_t f) { return f == MAB_KV_Q8 || f == MAB_KV_Q4 || f == MAB_KV_F16; }

// Verify sub-rows take two slot groups over quantized pools (the unquantized
// format's stage is too large for the two-buffer ring of the wide path) when
// some decode-path sequence has more than 16/G rows.
bool dec_wide_of(const mab_kv_layout* L, const mab_batch* B) {
  if (L->k_format == MAB_KV_F16 || L->v_format == MAB_KV_F16) return false;
  const int G = L->num_q_heads / L->num_kv_heads;
  for (int s = 0; s < B->num_seqs; ++s) {
    const int64_t q_len = (int64_t)B->q_start_host[s + 1] - B->q_start_host[s];
    if (q_len <= kMaxVerify && q_len > 16 / G) return true;  // a decode-path sequence past one slot group
  }
  return false;
}

int check_layout(const mab_kv_layout* L) {
  if (!L) return MAB_ERR_NULL;
  if (L->num_q_heads < 1 || L->num_kv_heads < 1 || L->num_q_heads % L->num_kv_heads) return MAB_ERR_SHAPE;
  if (L->head_dim < 32 || L->head_dim % 32 || L->page_size < 16 || L->page_size % 16) return MAB_ERR_SHAPE;
  if (L->num_pages < 1 || !fmt_ok(L->k_format) || !fmt_ok(L->v_format) || L->reserved) return MAB_ERR_SHAPE;
  if (L->head_dim != 64 && L->head_dim != 128) return MAB_ERR_UNSUPPORTED;
  if (L->num_q_heads / L->num_kv_heads > kMaxGroup) return MAB_ERR_UNSUPPORTED;
  if ((L->k_format == MAB_KV_F16) != (L->v_format == MAB_KV_F16)) return MAB_ERR_UNSUPPORTED;
  return MAB_OK;
}

struct HostPlan {
  int n_dec = 0, n_chunk = 0, n_chunk_items = 0, ch_target = 1;
  bool ch_splits = false;  // some chunk tile is cut into several splits
  int dec_units = 0, dec_wgs = 0, dec_range = 1, dec_pmax = 1;
  int dec_piece = 0;       // stages per piece with MAB_BATCH_INVARIANT, else 0
  bool dec_wide = false;   // some decode sub-row takes two slot groups
  int dec_seg_pieces = 1;  // pieces of the most cut decode segment
  int dec_slots = 1;       // (row, head) slots per decode partial
  int64_t n_slots = 0;
};

int debug_mode() {
  const char* e = getenv("MAB_DEBUG");
  return e && e[0] == '1' ? 1 : 0;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < 1)
    return 256;
  return cus;
}

int check_batch(const mab_kv_layout* L, const mab_batch* B, HostPlan* hp) {
  if (!B) return MAB_ERR_NULL;
  if (B->num_seqs < 0 || B->num_rows < 0 || B->max_pages_per_seq < 1 || (B->flags & ~MAB_BATCH_INVARIANT))
    return MAB_ERR_SHAPE;
  const int piece = (B->flags & MAB_BATCH_INVARIANT) ? kInvariantPiece : 0;
  if (B->num_seqs > kMaxSeqs) return MAB_ERR_UNSUPPORTED;
  if (B->num_seqs == 0) return B->num_rows == 0 ? MAB_OK : MAB_ERR_SHAPE;
  if (!B->q_start || !B->prefix_len || !B->block_table || !B->q_start_host || !B->prefix_len_host)
    return MAB_ERR_NULL;
  if (B->q_start_host[0] != 0 || B->q_start_host[B->num_seqs] != B->num_rows) return MAB_ERR_SHAPE;
  const bool wide = dec_wide_of(L, B);
  const int G = L->num_q_heads / L->num_kv_heads, hkv = L->num_kv_heads;
  const int cus = device_cus();
  const int ch_target = cus;  // resident chunk work-groups: one per compute unit
  int64_t items = 0, units = 0;
  int n_dec = 0, n_chunk = 0, max_ntok = 1;
  bool ch_splits = false;
  for (int s = 0; s < B->num_seqs; ++s) {
    const int64_t q_len = (int64_t)B->q_start_host[s + 1] - B->q_start_host[s];
    const int64_t prefix = B->prefix_len_host[s];
    if (q_len < 1 || prefix < 0) return MAB_ERR_SHAPE;
    const int64_t ctx = prefix + q_len;
    if (ctx > (int64_t)B->max_pages_per_seq * L->page_size || ctx > (int64_t)1 << 30) return MAB_ERR_SHAPE;
    if (is_chunk((int)q_len)) {
      const int tiles = chunk_tiles((int)q_len, hkv, G), f = chunk_split(tiles, ch_target);
      ++n_chunk;
      items += (int64_t)tiles * f;
      ch_splits |= f > 1;
    } else {
      const int T = dec_tokens((int)q_len, G, wide), nsub = dec_subrows((int)q_len, G, wide);
      for (int i = 0; i < nsub; ++i)
        units += (int64_t)hkv * dec_units_of((int)(prefix + std::min<int64_t>(q_len, (int64_t)(i + 1) * T)), piece);
      n_dec += nsub;
      max_ntok = std::max<int>(max_ntok, (int)std::min<int64_t>(q_len, T));
    }
  }
  if (items > (int64_t)1 << 30 || units > (int64_t)1 << 30) return MAB_ERR_UNSUPPORTED;
  if (!hp) return MAB_OK;
  hp->n_dec = n_dec;
  hp->n_chunk = n_chunk;
  hp->n_chunk_items = (int)items;
  hp->ch_target = ch_target;
  hp->ch_splits = ch_splits;
  hp->dec_units = (int)units;
  hp->dec_piece = piece;
  hp->dec_wide = wide;
  hp->dec_slots = max_ntok * G;
  if (units > 0) {
    // equal ranges, one per decode worker (a wave), as many as the device
    // holds at once (eight waves per compute unit: two 4-wave work-groups of
    // the decode kernel or one 8-wave work-group of the mixed kernel), fewer
    // for small batches: at least kMinWaveStages stages each
    // (with MAB_BATCH_INVARIANT: one piece per worker, as many workers as
    // pieces, the work-groups past the device's capacity dispatched as others
    // finish)
    const int nw = n_chunk > 0 ? kMixedWaves : kDecodeWaves;
    const int64_t max_workers = (int64_t)8 * cus;
    int64_t workers = std::min<int64_t>(max_workers, std::max<int64_t>(1, units / kMinWaveStages));
    int64_t range = ceil_div64(units, workers);
    if (piece > 0) range = piece;
    workers = ceil_div64(units, range);
    hp->dec_wgs = (int)ceil_div64(workers, nw);
    hp->dec_range = (int)range;
    // pieces per worker: one plus the segment starts strictly inside its range
    std::vector<int> pieces((size_t)workers, 1);
    int64_t x = 0;
    for (int s = 0; s < B->num_seqs; ++s) {
      const int q_len = B->q_start_host[s + 1] - B->q_start_host[s];
      if (is_chunk(q_len)) continue;
      for (int i = 0, T = dec_tokens(q_len, G, wide); i < dec_subrows(q_len, G, wide); ++i) {
      const int ctx = B->prefix_len_host[s] + std::min(q_len, (i + 1) * T);
      const int nst = dec_units_of(ctx, piece), nwork = dec_stages(ctx);
      for (int g = 0; g < hkv; ++g, x += nst) {
        if (x % range != 0) ++pieces[(size_t)(x / range)];
        hp->dec_seg_pieces = std::max<int>(hp->dec_seg_pieces, (int)((x + nwork - 1) / range - x / range + 1));
      }
      }
    }
    hp->dec_pmax = *std::max_element(pieces.begin(), pieces.end());
    hp->n_slots = (int64_t)workers * hp->dec_pmax;
  }
  return MAB_OK;
}

WsLayout plan_ws(const mab_kv_layout* L, const HostPlan& hp) {
  const int G = L->num_q_heads / L->num_kv_heads;
  const bool big = hp.n_dec > kArgDec || hp.n_chunk > kArgChunk;
  const int64_t chunk_rows_total = hp.ch_splits ? (int64_t)hp.n_chunk_items * chunk_heads(G) * chunk_rows(G) : 0;
  return ws_layout(hp.n_slots, hp.dec_slots, L->head_dim, chunk_rows_total, (int64_t)hp.n_dec * L->num_kv_heads,
                   big ? ws_tabs(hp.n_dec, hp.n_chunk).total : 0);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The launch-order tables in the kernel arguments (small batches).
void fill_arg_tabs(const mab_kv_layout* L, const mab_batch* B, AttnArgs* a) {
  const int G = L->num_q_heads / L->num_kv_heads, hkv = L->num_kv_heads;
  const bool wide = a->dec_wide != 0;
  int e = 0, c = 0, unit = 0, item = 0;
  for (int s = 0; s < B->num_seqs; ++s) {
    const int r0 = B->q_start_host[s], q_len = B->q_start_host[s + 1] - r0, prefix = B->prefix_len_host[s];
    if (is_chunk(q_len)) {
      a->tabs.ch_item[c] = item;
      a->tabs.ch_seq[c] = s;
      a->tabs.ch_r0[c] = r0;
      a->tabs.ch_qlen[c] = q_len;
      a->tabs.ch_prefix[c] = prefix;
      const int tiles = chunk_tiles(q_len, hkv, G), f = chunk_split(tiles, a->ch_target);
      a->tabs.ch_split[c] = f;
      item += tiles * f;
      ++c;
    } else {
      for (int i = 0, T = dec_tokens(q_len, G, wide); i < dec_subrows(q_len, G, wide); ++i, ++e) {
        const int t1 = std::min(q_len, (i + 1) * T);
        a->tabs.dec_unit[e] = unit;
        a->tabs.dec_seq[e] = s;
        a->tabs.dec_r0[e] = r0 + i * T;
        a->tabs.dec_ctx[e] = prefix + t1;
        a->tabs.dec_ntok[e] = t1 - i * T;
        unit += hkv * dec_units_of(prefix + t1, a->dec_piece);
      }
    }
  }
  a->tabs.dec_unit[e] = unit;
  a->tabs.ch_item[c] = item;
}

template <int KF, int VF>
void launch_append(const mab_kv_layout* L, const mab_batch* B, const void* kn, const void* vn, void* kp,
                   void* vp, hipStream_t st) {
  const int64_t n = 2LL * B->num_rows * L->num_kv_heads * (L->head_dim / 32);
  const int grid = (int)((n + 255) / 256);
  auto kernel = debug_mode() ? append_kernel<KF, VF, true> : append_kernel<KF, VF, false>;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, st, (const half_t*)kn, (const half_t*)vn, (uint8_t*)kp,
                     (uint8_t*)vp, B->q_start, B->prefix_len, B->block_table, B->num_seqs, B->num_rows,
                     B->max_pages_per_seq, L->num_kv_heads, L->head_dim, L->page_size, L->num_pages);
}

template <int NB, int KF, int VF, bool DBG, bool WIDE>
// ev0/ev1 (may be null): events that take the kernel's own start and end
// timestamps (hipExtLaunchKernel), for measurement.
void launch_attention_build(const AttnArgs& a, int grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.n_chunk_items > 0)
    hipExtLaunchKernelGGL((mixed_attention_kernel<NB, KF, VF, DBG, WIDE>), dim3(grid), dim3(64 * kMixedWaves), 0, st,
                          ev0, ev1, 0, a);
  else
    hipExtLaunchKernelGGL((decode_attention_kernel<NB, KF, VF, DBG, WIDE>), dim3(grid), dim3(64 * kDecodeWaves), 0,
                          st, ev0, ev1, 0, a);
}

template <int NB, int KF, int VF, bool DBG>
void launch_attention_dbg(const AttnArgs& a, int grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if constexpr (DecLayout<NB, KF, VF>::kWideOk) {
    if (a.dec_wide) {
      launch_attention_build<NB, KF, VF, DBG, true>(a, grid, st, ev0, ev1);
      return;
    }
  }
  launch_attention_build<NB, KF, VF, DBG, false>(a, grid, st, ev0, ev1);
}

// Debug mode takes instantiations of their own: the page-id checks stay out
// of the normal kernels' code.
template <int NB, int KF, int VF>
void launch_attention(const AttnArgs& a, int grid, hipStream_t st, bool debug, hipEvent_t ev0, hipEvent_t ev1) {
  if (debug) launch_attention_dbg<NB, KF, VF, true>(a, grid, st, ev0, ev1);
  else launch_attention_dbg<NB, KF, VF, false>(a, grid, st, ev0, ev1);
}

template <int NB>
void launch_attention_nb(const mab_kv_layout* L, const AttnArgs& a, int grid, hipStream_t st, bool dbg,
                         hipEvent_t ev0, hipEvent_t ev1) {
  if (L->k_format == MAB_KV_F16) launch_attention<NB, MAB_KV_F16, MAB_KV_F16>(a, grid, st, dbg, ev0, ev1);
  else if (L->k_format == MAB_KV_Q8 && L->v_format == MAB_KV_Q8) launch_attention<NB, MAB_KV_Q8, MAB_KV_Q8>(a, grid, st, dbg, ev0, ev1);
  else if (L->k_format == MAB_KV_Q8) launch_attention<NB, MAB_KV_Q8, MAB_KV_Q4>(a, grid, st, dbg, ev0, ev1);
  else if (L->v_format == MAB_KV_Q8) launch_attention<NB, MAB_KV_Q4, MAB_KV_Q8>(a, grid, st, dbg, ev0, ev1);
  else launch_attention<NB, MAB_KV_Q4, MAB_KV_Q4>(a, grid, st, dbg, ev0, ev1);
}

}  // namespace

extern "C" {

int32_t kv_block_bytes(int32_t format) {
  return format == MAB_KV_Q8 ? 34 : format == MAB_KV_Q4 ? 18 : format == MAB_KV_F16 ? 64 : 0;
}

int64_t kv_pool_bytes(const mab_kv_layout* layout, int32_t format) {
  if (!layout || !fmt_ok(format) || layout->num_pages < 1 || layout->num_kv_heads < 1 ||
      layout->page_size < 1 || layout->head_dim < 32 || layout->head_dim % 32)
    return -1;
  return (int64_t)layout->num_pages * layout->num_kv_heads * layout->page_size * (layout->head_dim / 32) *
         kv_block_bytes(format);
}

int64_t attention_workspace_bytes(const mab_kv_layout* layout, const mab_batch* batch) {
  int st = check_layout(layout);
  if (st) return -st;
  HostPlan hp;
  st = check_batch(layout, batch, &hp);
  if (st) return -st;
  return plan_ws(layout, hp).total;
}

int32_t kv_append_quant(const mab_kv_layout* layout, const mab_batch* batch, const void* k_new,
                        const void* v_new, void* k_pool, void* v_pool, void* stream) {
  int st = check_layout(layout);
  if (st) return st;
  st = check_batch(layout, batch, nullptr);
  if (st) return st;
  if (batch->num_rows == 0) return MAB_OK;
  if (!k_new || !v_new || !k_pool || !v_pool) return MAB_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool)) return MAB_ERR_ALIGN;
  hipStream_t hs = (hipStream_t)stream;
  const int kf = layout->k_format, vf = layout->v_format;
  if (kf == MAB_KV_F16) launch_append<MAB_KV_F16, MAB_KV_F16>(layout, batch, k_new, v_new, k_pool, v_pool, hs);
  else if (kf == MAB_KV_Q8 && vf == MAB_KV_Q8) launch_append<MAB_KV_Q8, MAB_KV_Q8>(layout, batch, k_new, v_new, k_pool, v_pool, hs);
  else if (kf == MAB_KV_Q8) launch_append<MAB_KV_Q8, MAB_KV_Q4>(layout, batch, k_new, v_new, k_pool, v_pool, hs);
  else if (vf == MAB_KV_Q8) launch_append<MAB_KV_Q4, MAB_KV_Q8>(layout, batch, k_new, v_new, k_pool, v_pool, hs);
  else launch_append<MAB_KV_Q4, MAB_KV_Q4>(layout, batch, k_new, v_new, k_pool, v_pool, hs);
  return hipGetLastError() == hipSuccess ? MAB_OK : MAB_ERR_HIP;
}

}  // extern "C"

namespace {

// The common body of mixed_attention_fwd and mixed_attention_fwd_noalloc.
int32_t attention_call(const mab_kv_layout* layout, const mab_batch* batch, const void* q, const void* k_pool,
                       const void* v_pool, float sm_scale, float* out, void* workspace, int64_t workspace_bytes,
                       void* stream, int32_t too_small, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
  int st = check_layout(layout);
  if (st) return st;
  HostPlan hp;
  st = check_batch(layout, batch, &hp);
  if (st) return st;
  if (!(sm_scale > 0.f) || !(sm_scale < INFINITY)) return MAB_ERR_UNSUPPORTED;  // logits kept unscaled
  if (batch->num_rows == 0) return MAB_OK;
  if (!q || !k_pool || !v_pool || !out || !workspace) return MAB_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) || !aligned16(workspace))
    return MAB_ERR_ALIGN;
  const WsLayout wl = plan_ws(layout, hp);
  if (workspace_bytes < wl.total) return too_small;

  char* ws = (char*)workspace;
  AttnArgs a;
  a.q = (const half_t*)q;
  a.k_pool = (const uint8_t*)k_pool;
  a.v_pool = (const uint8_t*)v_pool;
  a.q_start = batch->q_start;
  a.prefix_len = batch->prefix_len;
  a.block_table = batch->block_table;
  a.out = out;
  a.o_part = (float*)(ws + wl.o_off);
  a.ml_part = (float2*)(ws + wl.ml_off);
  a.ch_o = (float*)(ws + wl.cho_off);
  a.ch_ml = (float2*)(ws + wl.chml_off);
  a.dir = (DirEntry*)(ws + wl.dir_off);
  a.ws_tab = (int32_t*)(ws + wl.tab_off);
  a.num_seqs = batch->num_seqs;
  a.max_pages = batch->max_pages_per_seq;
  a.hq = layout->num_q_heads;
  a.hkv = layout->num_kv_heads;
  a.page_size = layout->page_size;
  a.n_dec = hp.n_dec;
  a.n_chunk = hp.n_chunk;
  a.n_chunk_items = hp.n_chunk_items;
  a.ch_target = hp.ch_target;
  a.dec_units = hp.dec_units;
  a.dec_piece = hp.dec_piece;
  a.dec_wide = hp.dec_wide ? 1 : 0;
  a.dec_range = hp.dec_range;
  a.dec_pmax = hp.dec_pmax;
  a.num_pages = layout->num_pages;
  a.dec_slots = hp.dec_slots;
  a.c = sm_scale * kLog2e;
  a.tabs_in_ws = hp.n_dec > kArgDec || hp.n_chunk > kArgChunk;
  hipStream_t hs = (hipStream_t)stream;
  if (a.tabs_in_ws) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, hs, a);
    if (hipGetLastError() != hipSuccess) return MAB_ERR_HIP;
  } else {
    fill_arg_tabs(layout, batch, &a);
  }
  const int grid = hp.n_chunk_items + hp.dec_wgs;
  const bool dbg = debug_mode();
  if (layout->head_dim == 64) launch_attention_nb<2>(layout, a, grid, hs, dbg, ev_start, ev_stop);
  else launch_attention_nb<4>(layout, a, grid, hs, dbg, ev_start, ev_stop);
  if (hipGetLastError() != hipSuccess) return MAB_ERR_HIP;
  if (hp.ch_splits) {
    hipLaunchKernelGGL(chunk_combine_kernel, dim3(hp.n_chunk_items * kChunkCombineGroups),
                       dim3(kChunkCombineThreads), 0, hs, a, layout->head_dim);
    if (hipGetLastError() != hipSuccess) return MAB_ERR_HIP;
  }
  if (hp.n_dec > 0) {
    const int nwg = hp.n_dec * layout->num_kv_heads * hp.dec_slots;
    const bool many = hp.dec_seg_pieces > kCombineWidePieces;
    if (layout->head_dim == 64) {
      if (many) hipLaunchKernelGGL((combine_kernel<32, 2, 2>), dim3(nwg * 2), dim3(32 * 8), 0, hs, a);
      else hipLaunchKernelGGL((combine_kernel<8, 2, 1>), dim3(nwg), dim3(8 * 16), 0, hs, a);
    } else {
      if (many) hipLaunchKernelGGL((combine_kernel<32, 4, 4>), dim3(nwg * 4), dim3(32 * 8), 0, hs, a);
      else hipLaunchKernelGGL((combine_kernel<8, 4, 1>), dim3(nwg), dim3(8 * 32), 0, hs, a);
    }
  }
  return hipGetLastError() == hipSuccess ? MAB_OK : MAB_ERR_HIP;
}

// The workspace of mixed_attention_fwd_noalloc: one array per device, held
// from the module's load on that device until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, taken once per device.
constexpr int64_t kScratchBytes = MAB_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// that device, with it current).
int32_t scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MAB_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MAB_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MAB_OK;
}

}  // namespace

extern "C" {

int32_t mixed_attention_fwd(const mab_kv_layout* layout, const mab_batch* batch, const void* q,
                            const void* k_pool, const void* v_pool, float sm_scale, float* out,
                            void* workspace, int64_t workspace_bytes, void* stream) {
  return attention_call(layout, batch, q, k_pool, v_pool, sm_scale, out, workspace, workspace_bytes, stream,
                        MAB_ERR_WORKSPACE);
}

int32_t mixed_attention_fwd_timed(const mab_kv_layout* layout, const mab_batch* batch, const void* q,
                                  const void* k_pool, const void* v_pool, float sm_scale, float* out,
                                  void* workspace, int64_t workspace_bytes, void* stream, void* kernel_start,
                                  void* kernel_stop) {
  return attention_call(layout, batch, q, k_pool, v_pool, sm_scale, out, workspace, workspace_bytes, stream,
                        MAB_ERR_WORKSPACE, (hipEvent_t)kernel_start, (hipEvent_t)kernel_stop);
}
int32_t mixed_attention_fwd_noalloc(const mab_kv_layout* layout, const mab_batch* batch, const void* q,
                                    const void* k_pool, const void* v_pool, float sm_scale, float* out,
                                    void* stream) {
  void* ws = nullptr;
  const int32_t st = scratch_of_current_device(&ws);
  if (st) return st;
  return attention_call(layout, batch, q, k_pool, v_pool, sm_scale, out, ws, kScratchBytes, stream,
                        MAB_ERR_SCRATCH);
}

int32_t mab_debug_status(int32_t reset) {
  int flag = 0;
  if (hipDeviceSynchronize() != hipSuccess) return -MAB_ERR_HIP;
  if (hipMemcpyFromSymbol(&flag, HIP_SYMBOL(g_mab_debug_flag), sizeof(flag)) != hipSuccess) return -MAB_ERR_HIP;
  if (reset) {
    const int zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_mab_debug_flag), &zero, sizeof(zero)) != hipSuccess) return -MAB_ERR_HIP;
  }
  return flag;
}

const char* mab_status_string(int32_t status) {
  switch (status) {
    case MAB_OK: return "ok";
    case MAB_ERR_NULL: return "a required pointer is NULL";
    case MAB_ERR_SHAPE: return "a layout or batch field breaks a stated rule";
    case MAB_ERR_UNSUPPORTED: return "shape outside the supported set";
    case MAB_ERR_WORKSPACE: return "workspace smaller than attention_workspace_bytes()";
    case MAB_ERR_ALIGN: return "a device buffer is not 16-byte aligned";
    case MAB_ERR_HIP: return "the HIP runtime refused a kernel launch";
    case MAB_ERR_QUOTA: return "client_quota: the client's pending requests are at their cap";
    case MAB_ERR_SCRATCH: return "the batch needs more workspace than the fixed scratch array of the no-allocation call";
    default: return "unknown status";
  }
}

}  // extern "C"
