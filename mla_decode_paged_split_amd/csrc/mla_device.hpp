// Device code for paged MLA decode on gfx950 (MI355X).
//
// What is computed (kernelindex amd-mixed-mla submission 689529, module
// constants and custom_kernel; submission 690201, the stage-1 / reduce pair):
// for each sequence b, its query token t and each of 16 heads h,
//   s_j = sm_scale * q_scale * kv_scale * <q[t,h,:576], kv[row_j,:576]>,
//   out[t,h,:512] = kv_scale * sum_j softmax(s)_j * kv[row_j,:512]
// over the rows row_j = kv_indices[i], i in [kv_indptr[b], kv_indptr[b+1]).
//
// Work split.  The rows of all sequences, concatenated in sequence order,
// form one row space of N rows.  It is cut into n_wg equal contiguous shares
// of C rows (C >= min_chunk, n_wg <= units): workgroup k owns rows
// [kC, (k+1)C).  A sequence that lies inside one share is finished by that
// workgroup; one that crosses shares is split, each piece writes a
// normalised float32 partial plus its log2-sum-exp, and the pieces are merged
// by a separate merge launch (or, optionally, by the last arriving workgroup).  This
// plays the role of the pages' metadata partitioner and persistent work list
// (submission 598454, get_mla_metadata_v1), but is recomputed from kv_indptr
// inside every launch, so nothing has to be rebuilt when lengths change.
//
// Inside a workgroup a piece is walked in tiles of 64 KV rows; wave w owns
// rows 16w..16w+15 of each tile.  Per tile a wave
//   1. has the 16 rows in VGPRs already: they were gathered through
//      kv_indices with 16-byte loads kDepth tiles earlier (a register ring,
//      so kDepth tiles per wave are in flight while it computes);
//   2. computes S^T = K . Q^T for its 16 rows with 16x16x32 MFMAs straight
//      from those registers (K rows on the M side, the 16 heads on the N
//      side, so every lane ends up owning one head) and copies the 512 V
//      bytes of each row into the shared LDS tile;
//   3. publishes its per-head tile max; after a barrier every wave applies the
//      same running max (log2 domain; the accumulator is rescaled only when
//      the max grows by more than 2^8), turns its scores into bf16 weights P
//      and publishes them;
//   4. after a second barrier computes O^T += V^T . P^T for its own 128 of the
//      512 output columns over all 64 rows.  V's rows must sit along the MFMA
//      K axis: each lane reads 8-row runs from LDS and interleaves them with
//      v_perm (widening fp8 to bf16, exact), or, for fp8 V in the register
//      ring, gets them from transposed reads (ds_read_b64_tr_b8).
// The waves own disjoint output columns, so finishing a piece only needs the
// per-head row sums of the 4 waves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mla {

constexpr int kHeads = 16;
constexpr int kQKDim = 576;
constexpr int kVDim = 512;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileRows = 64;             // KV rows per workgroup tile: 16 per wave
constexpr int kColsPerWave = kVDim / kWaves;  // 128 output columns per wave
constexpr int kSplitAlign = 32;           // share sizes are multiples of this
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;     // log2 growth of the running max tolerated before rescaling

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

enum class Dt : int { BF16 = 0, FP8 = 1 };

template <Dt KV>
struct KvLayout;

// fp8 rows: 576 bytes = 36 chunks of 16 bytes.  Lane (r, g) of a wave
// (r = lane % 16 its row, g = lane / 16) holds chunks 4j+g, j < 9, of row r;
// chunks j < 8 are the V part.
template <>
struct KvLayout<Dt::FP8> {
  static constexpr int kRowBytes = 576;
  static constexpr int kChunks = 9;
  static constexpr int kVChunks = 8;
  static constexpr int kVPitch = 528;  // LDS bytes per V row: 132 dwords, so row R starts 4R banks along
  static constexpr int kDepth = 3;     // tiles in flight per wave
};

// bf16 rows: 1152 bytes = 72 chunks; 18 per lane, 16 of them V.
template <>
struct KvLayout<Dt::BF16> {
  static constexpr int kRowBytes = 1152;
  static constexpr int kChunks = 18;
  static constexpr int kVChunks = 16;
  static constexpr int kVPitch = 1056;
  static constexpr int kDepth = 2;
};


// Q of a pass staged once per workgroup (fp8 KV only; bf16 KV keeps Q in
// each wave's registers): one row per token and head, bf16 (1152 B) or fp8
// (576 B) values, rows padded to 1168 B.
constexpr int kQPitch = 1168;

// Output staging at the finish, per wave and token, inside the tile buffers:
// 16 head rows of the wave's 128 columns, float32 (512 bytes) or bf16 (256
// bytes), each row padded by 16 bytes so that rows land on different banks.
constexpr int kOutPitchF32 = kColsPerWave * 4 + 16;
constexpr int kOutPitchBf16 = kColsPerWave * 2 + 16;
constexpr int kOutStageBytes = kHeads * kOutPitchF32;

// Two ways to stream the KV rows.  fp8 KV with one token per pass sends whole
// tiles into a ring of kSlots LDS tiles with direct-to-LDS loads: a tile is
// read by S^T in one step and by P.V in the next, so two of the four slots
// are in use and two tiles are in flight.  bf16 KV, and fp8 KV with two
// tokens per pass (whose second token's Q and accumulators leave no registers
// for the LDS ring's operands), hold the rows in a register ring and copy
// each tile's V part into one of two LDS buffers for P.V.
template <Dt KV, int QL>
constexpr bool lds_ring() {
  return KV == Dt::FP8 && QL == 1;
}
constexpr int kSlots = 4;
constexpr int kF8Row = 576;

// Sequences each thread reads in the first round trip, and the LDS table of
// their indptr values (what is left of the LDS beside the tile buffers).
template <Dt KV, int QL>
constexpr int scan_per_thread() {
  return lds_ring<KV, QL>() ? 2 : 4;
}
template <Dt KV, int QL>
constexpr int seq_table() {
  return scan_per_thread<KV, QL>() * kThreads;
}

template <Dt KV, int QL, bool kLds = lds_ring<KV, QL>()>
struct Smem;

// Register ring: the V parts of the current and the next tile, and the
// pass's Q (fp8 KV only; bf16 KV keeps Q in each wave's registers).
template <Dt KV, int QL>
struct alignas(16) Smem<KV, QL, false> {
  uint8_t v[2][kTileRows][KvLayout<KV>::kVPitch];
  uint8_t q[KV == Dt::FP8 ? QL * kHeads : 1][kQPitch];
  u32x2_t p[2][QL][kWaves][64];     // bf16 weights: token, wave, lane -> 4 rows of one head
  float mx[2][kWaves][QL][kHeads];  // per-wave tile max of each token and head
  float lsum[kWaves][QL][kHeads];
  int seq[seq_table<KV, QL>()][4];  // kv_indptr[b], kv_indptr[b+1], qo_indptr[b],
                                    // (tokens << 16) | last-page rows of the first sequences
  int differs[kWaves];  // per wave: some sequence's length differs from the first's
  int bmin;
  int bmax;
  int arrive;
  __device__ uint8_t* out_stage() { return &v[0][0][0]; }
  __device__ uint8_t* q_stage() { return &q[0][0]; }
};

// LDS ring: whole tiles (64 rows of 576 B).  Row R of a tile is at byte
// R * 576 of its slot and holds its 16-byte chunk c at position kpos(R, c),
// which spreads the fragment reads over the banks.  The pass's Q is staged in
// the last slot before that slot's first tile is loaded.
template <Dt KV, int QL>
struct alignas(16) Smem<KV, QL, true> {
  static_assert(KV == Dt::FP8 && QL == 1, "the LDS ring holds fp8 tiles for one token");
  uint8_t k[kSlots][kTileRows][kF8Row];
  u32x2_t p[2][QL][kWaves][64];
  float mx[2][kWaves][QL][kHeads];
  float lsum[kWaves][QL][kHeads];
  int seq[seq_table<KV, QL>()][4];
  int differs[kWaves];
  int bmin;
  int bmax;
  int arrive;
  __device__ uint8_t* out_stage() { return &k[0][0][0]; }
  __device__ uint8_t* q_stage() { return &k[kSlots - 1][0][0]; }
};
static_assert(sizeof(((Smem<Dt::BF16, 1>*)nullptr)->v) >= (size_t)kWaves * kOutStageBytes, "output staging fits");
static_assert(sizeof(((Smem<Dt::FP8, 2>*)nullptr)->v) >= (size_t)kWaves * kOutStageBytes, "output staging fits");
static_assert(sizeof(((Smem<Dt::FP8, 1>*)nullptr)->k[0]) >= (size_t)kWaves * kOutStageBytes, "output staging fits");
static_assert(sizeof(((Smem<Dt::FP8, 1>*)nullptr)->k[0]) >= (size_t)kHeads * kQPitch, "one token's Q fits a slot");
static_assert(sizeof(Smem<Dt::FP8, 1>) <= 160 * 1024 && sizeof(Smem<Dt::FP8, 2>) <= 160 * 1024 &&
                  sizeof(Smem<Dt::BF16, 1>) <= 160 * 1024,
              "LDS of one workgroup");

struct Args {
  const void* q;
  const void* kv;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last_page_len;  // [batch] rows in each sequence's last page, or null: pages full
  const float* q_scale;
  const float* kv_scale;
  float sm_scale;
  float logit_cap;    // 0: off
  uint16_t* out;      // bf16 bits [total_q, 16, 512]
  float* lse_out;     // [total_q, 16] natural-log sum-exp of each token's scores, or null
  float* part_o;      // [(2*units + batch*spec) * max_q_len, 16, 512]
  float* part_lse;    // [(2*units + batch*spec) * max_q_len, 16], log2 domain
  int32_t* counters;  // [batch] arrivals, then kGeoWords words: the split of the last attention launch
  int32_t batch;
  int32_t units;
  int32_t min_chunk;  // rows
  int32_t page_shift;  // log2(page size)
  int32_t max_q_len;   // query tokens per sequence at most
  int32_t causal;
  int32_t fused;
  int32_t q_cast;  // fp8 Q given as bf16: cast in the kernel (same rounding as mla_quantize_q_kernel)
  int32_t spec;    // pieces per sequence with partial slots of their own (0..kMaxSpec, see part_slot)
};

// ------------------------------------------------------------------ helpers

// Max / sum of x over lanes l and l ^ 16 (l ^ 32) of the wave, on the VALU:
// v_permlane16_swap / v_permlane32_swap of x with a copy of itself hands
// every lane the pair's two values (lower lane's first), where a shuffle
// would go through the LDS unit and cost a round trip there.  Written as one
// asm block: through the compiler builtin, given the same value twice, the
// swap's two results were folded into one and each lane combined its own
// value with itself.  The s_nop pairs cover the VALU-write-then-permlane
// hazard, which the compiler cannot see inside the block.
template <bool k32>
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  a = x;
  if constexpr (k32)
    asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "=&v"(b));
  else
    asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "=&v"(b));
}
// The same exchange for two independent values in one block, so the two
// chains overlap (separate volatile blocks keep their order and run back to
// back).
template <bool k32>
__device__ __forceinline__ void lane_pair2(float x0, float x1, float& a0, float& b0, float& a1, float& b1) {
  a0 = x0;
  a1 = x1;
  if constexpr (k32)
    asm volatile(
        "v_mov_b32 %1, %0\n\tv_mov_b32 %3, %2\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\t"
        "v_permlane32_swap_b32 %2, %3\n\ts_nop 1"
        : "+v"(a0), "=&v"(b0), "+v"(a1), "=&v"(b1));
  else
    asm volatile(
        "v_mov_b32 %1, %0\n\tv_mov_b32 %3, %2\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\t"
        "v_permlane16_swap_b32 %2, %3\n\ts_nop 1"
        : "+v"(a0), "=&v"(b0), "+v"(a1), "=&v"(b1));
}

// Max of x[q] over the four lanes l, l ^ 16, l ^ 32, l ^ 48, for each of N values.
template <int N>
__device__ __forceinline__ void quad_max(float (&x)[N]) {
  static_assert(N == 1 || N == 2, "one or two values");
  if constexpr (N == 1) {
    float a, b;
    lane_pair<false>(x[0], a, b);
    lane_pair<true>(fmaxf(a, b), a, b);
    x[0] = fmaxf(a, b);
  } else {
    float a0, b0, a1, b1;
    lane_pair2<false>(x[0], x[1], a0, b0, a1, b1);
    lane_pair2<true>(fmaxf(a0, b0), fmaxf(a1, b1), a0, b0, a1, b1);
    x[0] = fmaxf(a0, b0);
    x[1] = fmaxf(a1, b1);
  }
}

__device__ __forceinline__ float pair_max16(float x) {
  float a, b;
  lane_pair<false>(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_max32(float x) {
  float a, b;
  lane_pair<true>(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum16(float x) {
  float a, b;
  lane_pair<false>(x, a, b);
  return a + b;
}
__device__ __forceinline__ float pair_sum32(float x) {
  float a, b;
  lane_pair<true>(x, a, b);
  return a + b;
}

__device__ __forceinline__ float wave_max(float v) {
  v = pair_max32(v);
  v = pair_max16(v);
  for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = pair_sum32(v);
  v = pair_sum16(v);
  for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Two fp8 e4m3fn values (the low or the high 16 bits of `w`) -> two bf16,
// exact.  With a unit scale the scaled conversion is a plain widening.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  bf16x2_t r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight fp8 values (two dwords, byte k = element k) -> bf16x8.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t d0, uint32_t d1) {
  u32x4_t r;
  r[0] = fp8x2_to_bf16x2(d0, false);
  r[1] = fp8x2_to_bf16x2(d0, true);
  r[2] = fp8x2_to_bf16x2(d1, false);
  r[3] = fp8x2_to_bf16x2(d1, true);
  return __builtin_bit_cast(bf16x8_t, r);
}

// LDS read with an 8-bit transpose within each 16-lane group: lane
// 8h + i of the group receives, as byte e, byte i of the 8 bytes addressed by
// lane 2e + h of the group.  With the 16 lanes addressing 8 rows x two 8-byte
// column halves of a matrix, each lane gets one column over the 8 rows: the
// k-contiguous operand layout of a product whose k index runs over rows.
__device__ __forceinline__ u32x2_t lds_read_tr8(const uint8_t* p) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
  return u32x2_t{(uint32_t)r[0], (uint32_t)r[1]};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Stores of whole runs of results (bf16 rows, float32 partials and their
// lse, staged so that each store instruction covers whole lines) carry the
// non-temporal hint: nothing in the same launch reads them back, and lines
// that do not linger dirty in the L2 shorten the write-back at the end of the
// launch (the attention launch ran 0.8-1.1 us shorter on 64 x 8192 and
// 64 x 1024 batches than with plain stores).  Stores that write 16 bytes into
// each of 64 lines keep the plain form: with the hint the partial lines are
// not merged in the L2 (two causal tokens per pass ran ~21 us longer on a
// 64 x 8192 batch).
__device__ __forceinline__ void st_stream(const u32x4_t& v, uint16_t* dst) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
}
__device__ __forceinline__ void st_stream(const f32x4_t& v, float* dst) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(dst));
}

// Orders this wave's LDS stores before its later LDS loads of other lanes'
// data (a wave executes its LDS operations in order; this stops the compiler
// from moving them).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// bf16 -> fp8 e4m3fn, round to nearest even, non-saturating (magnitudes above
// 464, infinities and NaN give the NaN code with the input's sign).  Integer
// arithmetic on the bit fields, so the result does not depend on any
// hardware conversion mode.
__device__ __forceinline__ uint32_t bf16_to_e4m3fn(uint32_t x) {
  const uint32_t sign = (x >> 8) & 0x80u;
  const int e = (int)((x >> 7) & 0xFFu);
  const uint32_t m = x & 0x7Fu;
  if (e == 0xFF) return sign | 0x7Fu;
  int E = e - 127 + 7;  // e4m3 biased exponent
  if (E >= 1) {
    uint32_t m3 = m >> 4;
    const uint32_t rem = m & 0xFu;
    if (rem > 8u || (rem == 8u && (m3 & 1u))) ++m3;
    if (m3 == 8u) {
      m3 = 0;
      ++E;
    }
    if (E > 15 || (E == 15 && m3 == 7u)) return sign | 0x7Fu;
    return sign | ((uint32_t)E << 3) | m3;
  }
  // below 2^-6: units of 2^-9 (the e4m3 subnormal step)
  const int shift = 125 - e;  // significand (with hidden bit) is 8 bits wide
  if (e == 0 || shift > 9) return sign;  // bf16 subnormals and anything below 2^-10 round to zero
  const uint32_t sig = 0x80u | m;
  uint32_t n = sig >> shift;
  const uint32_t rem = sig & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (n & 1u))) ++n;
  return sign | n;  // n == 8 is the smallest normal, encoded the same way
}

// Eight bf16 Q values (four dwords) -> eight e4m3fn bytes, bit-identical to
// bf16_to_e4m3fn on each value.  The hardware conversion (low-word form,
// scale 1) agrees with it on every input except a positive NaN, to which it
// gives the negative NaN code; those bytes are patched to 0x7F without a
// branch.  Each pair goes through a named scalar: hipcc lowers
// __builtin_bit_cast of an ext-vector subscript to element 0 whatever the
// index.
__device__ __forceinline__ uint64_t bf16x8_to_e4m3fn(u32x4_t w) {
  typedef short short2v __attribute__((ext_vector_type(2)));
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t pair = w[i];
    const short2v o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(short2v{0, 0}, __builtin_bit_cast(bf16x2_t, pair),
                                                                1.0f, false);
    // bit 15 / 31 set where a half is a positive NaN: (h & 0x7fff) + 0x7f carries into bit 15, sign clear
    const uint32_t pn = ((pair & 0x7fff7fffu) + 0x007f007fu) & ~pair & 0x80008000u;
    const uint32_t fix = ((pn >> 15) & 1u) * 0xFFu | ((pn >> 31) * 0xFF00u);
    p[i] = ((__builtin_bit_cast(uint32_t, o) & 0xFFFFu) & ~fix) | (0x7F7Fu & fix);
  }
  return (uint64_t)(p[0] | (p[1] << 16)) | ((uint64_t)(p[2] | (p[3] << 16)) << 32);
}

// ---------------------------------------------------------------- partition

// The split works on index positions (pages): a share of C positions holds
// C pages, i.e. C * page_size rows except where a sequence's last page is
// part-filled.  C is a multiple of max(1, 32 / page_size) and at least
// min_chunk rows' worth of pages.
//
// Every sequence may also carry a fixed cost of kPieceCostRows rows:
// sequence b then occupies [kv_indptr[b] - base + cost * b, ... + its
// positions) of a "cost space" whose gaps belong to no one, and the shares
// cut that space.  Each piece a workgroup walks has a fixed price (a ring
// start, the Q load, the finish) of three to four tiles, so without the term a
// share that holds many sequence starts (many short sequences, or ragged
// lengths) takes that price many times while its neighbours take it once.
// The cost is left out (0) only where it cannot help: every sequence has the
// same length, at least kCostFreeMinRows rows, and that length and the share
// size divide one into the other, so every share holds whole sequences or
// whole fractions of one.
constexpr int kPieceCostRows = 256;
constexpr int kCostFreeMinRows = 1024;

struct Geo {
  int32_t base;   // kv_indptr[0]
  int32_t cost;   // positions of cost per sequence (0: none)
  int32_t total;  // extent of the split space: N index positions + cost * batch
  int32_t chunk;  // C positions per workgroup share
  int32_t n_wg;   // shares in use (>= 1)
};
constexpr int kGeoWords = 8;  // the attention launch's Geo, kept for the merge launch after the counters

// Share size: ceil(total / units) rounded up to align (a power of two), at
// least min_pos.  Totals fit int32 (the pool rows do), so the divisions are
// 32-bit unsigned ones.
__device__ __forceinline__ int32_t share_size(int32_t total, int units, int align, int min_pos) {
  const uint32_t c = ((uint32_t)total + (uint32_t)units - 1u) / (uint32_t)units;
  const int32_t r = (int32_t)((c + (uint32_t)align - 1u) & ~((uint32_t)align - 1u));
  return r < min_pos ? min_pos : r;
}

__device__ __forceinline__ int32_t share_count(int32_t total, int32_t chunk) {
  const int32_t n = (int32_t)(((uint32_t)total + (uint32_t)chunk - 1u) / (uint32_t)chunk);
  return n < 1 ? 1 : n;
}

// The split with no cost term, from kv_indptr[0] and kv_indptr[batch].
__device__ __forceinline__ Geo cost_free_geo(int32_t ip_first, int32_t ip_last, int units, int min_chunk, int sh) {
  Geo g;
  g.base = ip_first;
  g.cost = 0;
  g.total = ip_last - g.base;
  g.chunk = share_size(g.total, units, max(1, kSplitAlign >> sh), max(1, min_chunk >> sh));
  g.n_wg = share_count(g.total, g.chunk);
  return g;
}

// The split: the cost-free one g0 when every sequence has the same length
// (uniform_len >= 0; -1 if they differ), at least kCostFreeMinRows rows, that
// divides the share size or is divided by it; else one with the cost term.
__device__ __forceinline__ Geo make_geo(const Geo& g0, int batch, int units, int min_chunk, int sh, int uniform_len) {
  const bool long_seqs = uniform_len >= max(1, kCostFreeMinRows >> sh);
  if (long_seqs && (uniform_len % g0.chunk == 0 || g0.chunk % uniform_len == 0)) return g0;
  Geo g = g0;
  g.cost = max(1, kPieceCostRows >> sh);
  g.total += g.cost * batch;
  g.chunk = share_size(g.total, units, max(1, kSplitAlign >> sh), max(1, min_chunk >> sh));
  g.n_wg = share_count(g.total, g.chunk);
  return g;
}

// Share slot of the i-th piece of a sequence occupying [st, en) of the split
// space (en > st): workgroup k has two, 2k for the piece of its first
// sequence and 2k+1 for the piece of its last one; a sequence that starts
// exactly at a share boundary is the first sequence of that share.  (The
// partial buffers put the per-sequence slots of part_slot before these.)
__device__ __forceinline__ int piece_slot(int st, int chunk, int i) {
  const int k1 = st / chunk;
  return i == 0 ? 2 * k1 + (st != k1 * chunk ? 1 : 0) : 2 * (k1 + i);
}

__device__ __forceinline__ int piece_count(int st, int en, int chunk) {
  return (en - 1) / chunk - st / chunk + 1;
}

// Partial slot of piece i of sequence b.  The first `spec` pieces of every
// sequence have slots of their own, b * spec + i, which the merge launch can
// load before it has read the split (its first round trip); the others
// follow them, in the slots of their workgroup shares (piece_slot).  The
// library chooses spec = min(units / batch, kMaxSpec) (the pieces of a
// sequence when every sequence has the same length) where units >= 2 * batch,
// else 0.
constexpr int kMaxSpec = 16;
__device__ __forceinline__ int part_slot(int b, int i, int st, int chunk, int spec, int batch) {
  return i < spec ? b * spec + i : batch * spec + piece_slot(st, chunk, i);
}

// ------------------------------------------------------------------- merge

// Pieces 0..kMaxSpec-1 of one head, loaded by the merge launch before it knows
// how many the sequence has: lane l's 8 columns of each, and lane i's lse of
// piece i.
struct MergePre {
  f32x4_t a[kMaxSpec], b[kMaxSpec];
  float lse;
};

// One wave merges the S partials of one head:
//   out[h,:] = sum_i 2^(lse_i - M) o_i[h,:] / sum_i 2^(lse_i - M),  M = max_i lse_i,
// lse multiplied by lse_mul to reach the log2 domain.  Lane i < 64 of a chunk
// owns piece i's lse (max and weights by wavefront shuffles); lane l owns the
// 8 output columns 8l..8l+7 and walks the pieces with the weights broadcast
// by lane shuffles.  The first batch of partial loads is issued before the
// lse arithmetic so a merge of a few pieces costs about one memory round trip.
// A piece of weight 0 (lse = -inf) is selected out rather than multiplied, so
// whatever its partial row holds (an empty shard's 0/0) cannot reach the sum;
// a NaN lse (NaN inputs) gives a NaN weight and a NaN result.
// With lse_dst, lane 0 also stores the merged natural-log sum-exp,
// (M + log2 sum_i 2^(lse_i - M)) ln 2, or -inf when every piece is empty.
// kPre: all S <= kMaxSpec pieces are already loaded in *pre (the same
// arithmetic in one pass; a mix of loaded and preloaded pieces would join the
// two paths on values still in flight, and the compiler waits for them there).
template <bool kPre = false, class SlotFn>
__device__ void merge_head_wave(const float* __restrict__ part_o, const float* __restrict__ part_lse, int S,
                                SlotFn slot_of, float lse_mul, int h, uint16_t* __restrict__ out_head,
                                float* __restrict__ lse_dst, const MergePre* pre = nullptr) {
  const int lane = threadIdx.x & 63;
  constexpr int kBatch = 8;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY;
  float wsum = 0.f;
  for (int i0 = 0; i0 < S; i0 += 64) {
    const int n = min(64, S - i0);
    if constexpr (kPre) {  // S <= kMaxSpec: one chunk, every piece in *pre
      const float v = (lane < n) ? pre->lse * lse_mul : -INFINITY;
      M = wave_max(v);
      const float wt = (v == -INFINITY) ? 0.f : fast_exp2(v - M);
      wsum = wave_sum(wt);
#pragma unroll
      for (int u = 0; u < kMaxSpec / 2; ++u)
        if (u < n) {
          const float wj = __shfl(wt, u);
          acc0 += wj != 0.f ? wj * pre->a[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
          acc1 += wj != 0.f ? wj * pre->b[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      if (n > kMaxSpec / 2) {
#pragma unroll
        for (int u = kMaxSpec / 2; u < kMaxSpec; ++u)
          if (u < n) {
            const float wj = __shfl(wt, u);
            acc0 += wj != 0.f ? wj * pre->a[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc1 += wj != 0.f ? wj * pre->b[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
      }
      break;
    }
    f32x4_t a[kBatch], b[kBatch];
    float v;
    {
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (u < n) {
          const f32x4_t* src =
              reinterpret_cast<const f32x4_t*>(part_o + ((size_t)slot_of(i0 + u) * kHeads + h) * kVDim + lane * 8);
          a[u] = src[0];
          b[u] = src[1];
        }
      v = (lane < n) ? part_lse[slot_of(i0 + lane) * kHeads + h] * lse_mul : -INFINITY;
    }
    const float m_new = fmaxf(M, wave_max(v));
    if (m_new != M) {  // rescale what earlier chunks accumulated (uniform across the wave)
      const float r = (M == -INFINITY) ? 0.f : fast_exp2(M - m_new);
      acc0 *= r;
      acc1 *= r;
      wsum *= r;
      M = m_new;
    }
    const float wt = (v == -INFINITY) ? 0.f : fast_exp2(v - M);
    wsum += wave_sum(wt);
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (u < n) {
        const float wj = __shfl(wt, u);
        acc0 += wj != 0.f ? wj * a[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1 += wj != 0.f ? wj * b[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    for (int j0 = kBatch; j0 < n; j0 += kBatch) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (j0 + u < n) {
          const f32x4_t* src = reinterpret_cast<const f32x4_t*>(
              part_o + ((size_t)slot_of(i0 + j0 + u) * kHeads + h) * kVDim + lane * 8);
          a[u] = src[0];
          b[u] = src[1];
        }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (j0 + u < n) {
          const float wj = __shfl(wt, j0 + u);
          acc0 += wj != 0.f ? wj * a[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
          acc1 += wj != 0.f ? wj * b[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
  }
  const float inv = wsum == 0.f ? 0.f : 1.0f / wsum;
  u32x4_t pk;
  pk[0] = pack_bf16x2(acc0[0] * inv, acc0[1] * inv);
  pk[1] = pack_bf16x2(acc0[2] * inv, acc0[3] * inv);
  pk[2] = pack_bf16x2(acc1[0] * inv, acc1[1] * inv);
  pk[3] = pack_bf16x2(acc1[2] * inv, acc1[3] * inv);
  st_stream(pk, out_head + lane * 8);
  if (lse_dst != nullptr && lane == 0) *lse_dst = wsum == 0.f ? -INFINITY : (M + fast_log2(wsum)) * kLn2;
}

// ------------------------------------------------------------- zero output

__device__ __forceinline__ void zero_row_by_thread(uint16_t* out_row) {
  u32x4_t z = {0u, 0u, 0u, 0u};
  u32x4_t* p = reinterpret_cast<u32x4_t*>(out_row);
  for (int i = 0; i < kHeads * kVDim * 2 / 16; ++i) p[i] = z;
}

// --------------------------------------------------------------- one piece

// Row `pr` of a piece that starts at index position ip0 and has nrows rows
// lives in page kv_indices[ip0 + pr / page_size], slot pr % page_size
// (page_size = 2^sh), i.e. pool row page * page_size + slot.  Rows at or past
// nrows stand for the piece's last row instead: always valid, and the ring's
// loads past the end (issued in the last steps, never used) then read what
// the last tile has just brought into the cache instead of waiting on memory.
// The page load and the row composition are separate so that the ring can
// keep the raw page index in flight and compose the row only when it issues
// the tile's loads (using a loaded value at once would wait for it).
__device__ __forceinline__ int piece_page(const int32_t* __restrict__ kv_indices, int ip0, int nrows, int pr,
                                          int sh) {
  return kv_indices[ip0 + ((pr < nrows ? pr : nrows - 1) >> sh)];
}

__device__ __forceinline__ int page_row(int page, int nrows, int pr, int sh) {
  return (page << sh) | ((pr < nrows ? pr : nrows - 1) & ((1 << sh) - 1));
}

// The register ring of one piece: the rows of D tiles in flight (tile t in
// slot t % D) and the row indices of the next D tiles.  Lane (c16, g) of wave
// w owns row 16w + c16 of every 64-row tile and 16-byte chunks 4j + g of it.
// Tiles in flight per wave: the layout's depth, one less when two tokens
// share the walk.  Two tokens double the products and the softmax, so that
// walk is bound by its arithmetic rather than by memory, and the registers a
// deeper ring holds serve the compiler's schedule better (fp8 Q: 1.3 us
// shorter on a 64 x 8192 batch with a ring of two tiles than of three; bf16 Q
// needs the room for its second token's 72 registers of Q).  Over bf16 KV
// that leaves one tile of 72 registers (a second one spilled).
template <Dt QT, Dt KT, int QL>
constexpr int ring_depth() {
  return QL > 1 ? KvLayout<KT>::kDepth - 1 : KvLayout<KT>::kDepth;
}

template <Dt KT, int Depth>
struct Ring {
  static constexpr int D = Depth;
  static constexpr bool kNext = true;
  u32x4_t dat[D][KvLayout<KT>::kChunks];
  int first[D];  // pages of tiles 0..D-1
  int next[D];   // pages of tiles D..2D-1, then of each slot's next refill
};

// fp8 KV: the page index of the tile each LDS slot receives next (tile t
// goes to slot t % kSlots).  first / next hold tiles 0..3 and 4..7 when a
// piece starts; after the first three tiles are requested, slot j's entry is
// the next tile it receives.
struct LdsRing {
  static constexpr int D = kSlots;
  static constexpr bool kNext = false;  // the pages of tiles 4..6 are loaded as tiles 0..2 go out
  int first[D];
};

template <Dt QT, Dt KT, int QL>
using RingOf = std::conditional_t<lds_ring<KT, QL>(), LdsRing, Ring<KT, ring_depth<QT, KT, QL>()>>;

// Position of chunk c of tile row R inside its row.  With a = (R >> 2) & 3,
// the chunk index is xor-ed with a, and for the 32 V chunks also with
// (a & 1) << 3 (a 128-byte move that keeps them inside the first 32).  An
// S^T fragment read (16 rows, one chunk each) then hits 16 different
// 16-byte bank groups, and a P.V read (rows 4 apart, 128 contiguous bytes
// each) puts the two 16-lane groups served together 128 bytes apart.  The
// map is its own inverse on each row.
__device__ __forceinline__ int kpos(int R, int c) {
  const int a = (R >> 2) & 3;
  return c ^ a ^ (c < 32 ? (a & 1) << 3 : 0);
}

// Direct-to-LDS loads of this wave's 16 rows of a tile into `slot`: tile
// row R = 16w + r goes to slot + R * 576, chunk c of it to position
// kpos(R, c) (kpos(16w + r, c) == kpos(r, c)).  The wave's rows are 576 sixteen-byte units of the slot;
// instruction i fills units 64i .. 64i + 63 (lane l unit 64i + l), so each
// instruction writes 1 KB of LDS and, for rows that are neighbours in the
// pool, reads 1 KB of contiguous memory: whole lines, with the non-temporal
// hint so nothing lingers in the caches.  Every lane of every instruction
// is active (an exec-masked block would make the compiler assume it may be
// skipped and drain every load in flight where it waits for the page
// indices).  Lane l's row of instruction i is fetched from the lane that
// holds it (row_v: lane r < 16 holds the pool row of the wave's row r) with
// ds_bpermute; the per-lane source lane and chunk offset are constants.
struct DmaLanes {
  int src[9];       // ds_bpermute byte address of the lane holding this lane's row
  uint32_t off[9];  // byte offset of this lane's chunk in its row
};

__device__ __forceinline__ DmaLanes dma_lanes() {
  DmaLanes d;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int u = 64 * i + lane;
    const int r = u / 36;
    d.src[i] = r * 4;
    d.off[i] = (uint32_t)(kpos(r, u - r * 36) << 4);  // the chunk stored at this position
  }
  return d;
}

// The rows of the 9 instructions, fetched ahead of the loads (the exchange
// goes through the LDS unit; fetched well before the loads, its latency is
// hidden and the loads need no wait of their own).
struct DmaRows {
  uint32_t row[9];
};
__device__ __forceinline__ DmaRows dma_rows(int row_v, const DmaLanes& dl) {
  DmaRows r;
#pragma unroll
  for (int i = 0; i < 9; ++i) r.row[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(dl.src[i], row_v);
  return r;
}
// Instruction i of a tile's loads; `dst` is this wave's 16 rows of the slot.
__device__ __forceinline__ void dma_one(const void* kv, uint8_t* dst, const DmaRows& r, const DmaLanes& dl, int i) {
  const uint8_t* src = reinterpret_cast<const uint8_t*>(kv) + (size_t)r.row[i] * kF8Row + dl.off[i];
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                   reinterpret_cast<__attribute__((address_space(3))) void*>((uintptr_t)(dst + i * 1024)),
                                   16, 0, 2 /* nt */);
}
__device__ __forceinline__ void dma_issue(const void* kv, uint8_t* dst, const DmaRows& r, const DmaLanes& dl) {
#pragma unroll
  for (int i = 0; i < 9; ++i) dma_one(kv, dst, r, dl, i);
}
// Vector-memory instructions per tile: its 9 loads, then one page-index load
// (of the tile 4 later into the same slot).  Every tile, the first ones
// included, is issued in this pattern, so one wait count serves every step.
constexpr int kDmaOps = 9;
constexpr int kTileOps = kDmaOps + 1;

// Wait until at most n vector-memory operations of this wave are in flight
// (the direct-to-LDS loads land in LDS when they leave this count).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits for this wave's LDS operations but not for
// its direct-to-LDS loads in flight (__syncthreads would: they write LDS).
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Fetch the ring's starting page indices for a piece of nrows rows beginning
// at index position ip0.
template <class R>
__device__ __forceinline__ void issue_ring_indices(const int32_t* __restrict__ kv_indices, int ip0, int nrows,
                                                   int sh, R& r) {
  constexpr int D = R::D;
  const int my_row = 16 * (threadIdx.x >> 6) + (threadIdx.x & 15);
#pragma unroll
  for (int k = 0; k < D; ++k) r.first[k] = piece_page(kv_indices, ip0, nrows, k * kTileRows + my_row, sh);
  if constexpr (R::kNext) {
#pragma unroll
    for (int k = 0; k < D; ++k) r.next[k] = piece_page(kv_indices, ip0, nrows, (k + D) * kTileRows + my_row, sh);
  }
}

// Start the loads of the ring's first D tiles (in the steady state's slot
// order, kept by scheduling barriers so the loop's wait counts stay exact).
// Rows at or past nrows load the piece's last row (never used).
template <Dt KT, class R>
__device__ __forceinline__ void issue_ring_rows(const void* kv, int nrows, int sh, R& r) {
  using L = KvLayout<KT>;
  constexpr int D = R::D;
  const int g = (threadIdx.x & 63) >> 4;
  const int my_row = 16 * (threadIdx.x >> 6) + (threadIdx.x & 15);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < D; ++k) {
    const int row = page_row(r.first[k], nrows, k * kTileRows + my_row, sh);
    const uint8_t* src = reinterpret_cast<const uint8_t*>(kv) + (size_t)row * L::kRowBytes + g * 16;
#pragma unroll
    for (int j = 0; j < L::kChunks; ++j) r.dat[k][j] = *reinterpret_cast<const u32x4_t*>(src + j * 64);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pass over a piece: its rows, the query tokens it serves in this pass
// and where their results go.
template <int QL>
struct Piece {
  int ip0;        // first index position
  int nrows;      // rows of the piece
  int t0;         // query row of the pass's first token
  int ntok;       // tokens in this pass, 1..QL
  int lim[QL];    // rows (from the piece start) token j sees: <= nrows, <= 0 for none
  int slot;       // partial row of token j is slot + j (unused when complete)
  bool complete;  // the piece is the whole sequence: write bf16 rows
  bool last;      // no other pass follows in this workgroup (one token: stream the results out)
};

// Score transform, raw dot product -> log2-domain logit: sc * c_score, or
// with the soft-cap cap * tanh(sc * c_nat / cap) * log2(e), computed as
// k2 * (1 - 2 / (2^(k1 sc) + 1)) with k1 = 2 log2(e) c_nat / cap and
// k2 = cap log2(e) (the limits +-1 come out exactly when 2^(k1 sc)
// overflows or underflows).
struct Logit {
  float c_score;
  float k1;
  float k2;
  // The cap is a kernel form of its own, not a runtime branch: given a
  // runtime choice the compiler evaluated both forms for every score (eight
  // more exp2 and reciprocals per step with two tokens) and selected.
  template <bool kCap>
  __device__ __forceinline__ void apply(const f32x4_t& sc, float (&y)[4]) const {
    if constexpr (kCap) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(sc[i] * k1);
        y[i] = k2 * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = sc[i] * c_score;
    }
  }
};

// Attention of the pass's query tokens over the rows of one piece.  All 256
// threads take part; the workgroup writes either the final bf16 rows
// (complete) or the float32 partials.  kGeneral = false is the plain decode
// (pages of one row, no soft-cap), with both compiled out of the loop.
template <Dt QT, Dt KT, int QL, bool kGeneral, bool kCap, class RingT>
__device__ void attend_piece(const Args& a, Smem<KT, QL>& sm, const Piece<QL>& pc, const Logit logit,
                             float out_mul, RingT& ring, const DmaLanes& dl) {
  using L = KvLayout<KT>;
  constexpr int D = RingT::D;
  constexpr bool kLds = lds_ring<KT, QL>();
  // (not const: the LDS ring re-derives them once the first tiles' loads are out)
  int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int c16 = lane & 15;
  int g = lane >> 4;
  const int sh = kGeneral ? a.page_shift : 0;
  int my_row = 16 * w + c16;  // this lane's row within a tile (for loads)
  // LDS ring: the rows of the tile whose loads the next step issues (dl: the
  // per-lane constants of the tile loads), this wave's 16 rows in a slot (the
  // wave index made a scalar once) and the next S^T's K fragments
  [[maybe_unused]] DmaRows pend;
  [[maybe_unused]] const int wrow_bytes = 16 * __builtin_amdgcn_readfirstlane(w) * kF8Row;
  [[maybe_unused]] u32x4_t kcur[KvLayout<KT>::kChunks];

  // Q as the B operand of S^T = K . Q^T (lane holds head c16).  A k-step takes
  // 8 values per lane; for fp8 KV a 16-byte chunk feeds two k-steps, for bf16
  // KV one.  Q is read with the same d mapping as the K chunks.  Tokens past
  // ntok read the first token's row (their results are never written).
  constexpr int kSteps = kQKDim / 32;  // 18
  bf16x8_t qb[QL][QT == Dt::BF16 ? kSteps : 1];
  uint64_t q8[QL][QT == Dt::FP8 ? kSteps : 1];
  if constexpr (KT == Dt::FP8) {
    // Q goes through LDS: the workgroup loads each token's 16 rows once (16-byte
    // pieces over all 256 threads) instead of every wave loading all of them,
    // so 4x fewer requests sit in front of the tiles.  Order: Q loads, the
    // first tiles, then (register ring) Q into LDS (cast to fp8 there when
    // fp8 Q is given as bf16), a barrier once tile 0 has landed, and each
    // wave's fragments from LDS.
    const bool src16 = (QT == Dt::BF16) || a.q_cast;  // the source holds bf16 values
    constexpr int kChunks16 = kHeads * kQKDim * 2 / 16;  // 1152 sixteen-byte pieces of a bf16 Q token
    constexpr int kPer = (kChunks16 + kThreads - 1) / kThreads;  // 5
    const int nchunks = src16 ? kChunks16 : kChunks16 / 2;
    const int per_head = src16 ? kQKDim * 2 / 16 : kQKDim / 16;  // 72 or 36
    [[maybe_unused]] u32x4_t stage[QL][kPer];
    if constexpr (kLds) {
      // The ring's page indices are in before anything else goes out.  For
      // the first piece they were requested before the start's barriers and
      // have long arrived; a later piece needs them for its first tile
      // anyway.  Without this wait the compiler, joining the two paths,
      // cannot count which loads the second tile's indices are behind and
      // waits for all of them, the first tile's own loads included.
      wait_vm<0>();
    }
    // bf16 Q in the LDS ring: straight into LDS slot 3 with direct-to-LDS
    // loads, so that no register has to wait for it behind the tiles' loads
    // (a store of loaded Q to LDS after them makes the compiler wait for
    // every tile load, tile 1's included: the first step would start only
    // once tiles 0 and 1 are in).  Staging chunk p (16 bytes) is column
    // p % 73 of head row p / 73 (1168-byte pitch); columns past the row's end
    // and rows past the 16th fetch the row's last chunk and land in unused
    // space of the slot.  fp8 Q keeps the register path (it is cast to fp8
    // on the way when given as bf16; cast after a direct-to-LDS load, in
    // LDS, it came out 0.4 us slower on the 64 x 8192 batch).
    constexpr bool kQDma = kLds && QT == Dt::BF16;
    if constexpr (kQDma) {
      constexpr int kQPitchChunks = kQPitch / 16;                                       // 73
      constexpr int kQDmaOps = (kHeads * kQPitchChunks + kThreads - 1) / kThreads;      // 5 per wave
      static_assert(kQDmaOps * kThreads * 16 <= kTileRows * kF8Row, "Q staging fits a slot");
      constexpr int ncol = kQKDim * 2 / 16;  // 72 chunks per head row
      const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q) + (size_t)pc.t0 * kHeads * kQKDim * 2;
      const int wq = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
      for (int ii = 0; ii < kQDmaOps; ++ii) {
        const int j = ii * kWaves + wq;  // this wave's 1 KB of the staging
        const int pch = j * 64 + lane;
        const int row = min(pch / kQPitchChunks, kHeads - 1);
        const int col = min(pch - (pch / kQPitchChunks) * kQPitchChunks, ncol - 1);
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(qsrc + (size_t)row * ncol * 16 + col * 16),
            reinterpret_cast<__attribute__((address_space(3))) void*>((uintptr_t)(sm.q_stage() + j * 1024)), 16,
            0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      if constexpr (kQDma) break;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(a.q) +
                           (size_t)(pc.t0 + (q < pc.ntok ? q : 0)) * kHeads * kQKDim * (src16 ? 2 : 1);
      // every thread issues all kPer loads (index clamped; surplus ones are not
      // written to LDS): the compiler counts only unconditional loads when it
      // works out how long the ring's row addresses must wait for their page
      // indices, and a load inside a branch would make the third tile's rows
      // wait for the first Q load
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int c = min((int)threadIdx.x + i * kThreads, nchunks - 1);
        stage[q][i] = *reinterpret_cast<const u32x4_t*>(src + (size_t)c * 16);
      }
    }
    if constexpr (kLds && !kQDma) __builtin_amdgcn_sched_barrier(0);  // every Q load before the tiles' loads
    if constexpr (kLds) {
      // tiles 0 and 1 now (ring.first[j] becomes the page of the next tile
      // slot j receives: 4 and 5); tile 2 goes out during the first step's
      // S^T, as every later tile goes out during the S^T of the step after
      // the one that freed its slot
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        dma_issue(a.kv, &sm.k[k][0][0] + wrow_bytes,
                  dma_rows(page_row(ring.first[k], pc.nrows, k * kTileRows + my_row, sh), dl), dl);
        ring.first[k] = piece_page(a.kv_indices, pc.ip0, pc.nrows, (k + kSlots) * kTileRows + my_row, sh);
      }
      pend = dma_rows(page_row(ring.first[2], pc.nrows, 2 * kTileRows + my_row, sh), dl);
      // Q is in (behind it: the two tiles' loads and two page loads)
      if constexpr (!kQDma) wait_vm<2 * kTileOps>();
      // The lane indices again, from a copy the compiler cannot see through:
      // the per-lane addresses of the steps that follow derive from them, and
      // would otherwise be computed once before the piece loop, on the way to
      // these loads; now they are computed while the loads fly.
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      lane = tid & 63;
      c16 = lane & 15;
      g = lane >> 4;
      my_row = 16 * w + c16;
    } else {
      issue_ring_rows<KT>(a.kv, pc.nrows, sh, ring);
    }
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      if constexpr (kQDma) break;  // staged by its direct-to-LDS loads
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int c = threadIdx.x + i * kThreads;
        if (c < nchunks) {
          const int h = c / per_head;
          const int off = (c - h * per_head) * 16;  // byte offset in the source row
          uint8_t* dst = sm.q_stage() + (q * kHeads + h) * kQPitch;
          if (QT == Dt::FP8 && a.q_cast)
            *reinterpret_cast<uint64_t*>(dst + off / 2) = bf16x8_to_e4m3fn(stage[q][i]);
          else
            *reinterpret_cast<u32x4_t*>(dst + off) = stage[q][i];
        }
      }
    }
    if constexpr (kLds) {
      wait_vm<kTileOps + 1>();  // Q and tile 0 are in LDS (after them: tile 1's loads and two page loads)
      lds_barrier();
    } else {
      __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      const uint8_t* row = sm.q_stage() + (q * kHeads + c16) * kQPitch;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int d0 = ((s >> 1) * 4 + g) * 16 + (s & 1) * 8;
        if constexpr (QT == Dt::BF16)
          qb[q][s] = *reinterpret_cast<const bf16x8_t*>(row + d0 * 2);
        else
          q8[q][s] = *reinterpret_cast<const uint64_t*>(row + d0);
        // two tokens of bf16 Q (144 registers): Q lives in the accumulation
        // registers, which the products read directly (held in the vector
        // registers, it would be spilled there and copied back before every
        // product).  fp8 Q (72 registers) fits in the vector registers.
        if constexpr (QL > 1 && QT == Dt::BF16) asm volatile("" : "+a"(qb[q][s]));
      }
    }
  } else {
    // bf16 KV (bf16 Q only): every wave loads the whole Q straight into its registers
    static_assert(QT == Dt::BF16, "fp8 Q is paired with fp8 KV only");
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      const size_t qrow = ((size_t)(pc.t0 + (q < pc.ntok ? q : 0)) * kHeads + c16) * kQKDim;
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
        qb[q][s] = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const uint16_t*>(a.q) + qrow + (s * 4 + g) * 8);
    }
    // the ring's rows go out after Q (their page indices were fetched before the piece began)
    issue_ring_rows<KT>(a.kv, pc.nrows, sh, ring);
  }

  // tiles up to the furthest row any token of the pass sees
  int maxlim = 0;
#pragma unroll
  for (int q = 0; q < QL; ++q) maxlim = max(maxlim, pc.lim[q]);
  const int T = (maxlim + kTileRows - 1) / kTileRows;
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(a.kv);

  // the ring is primed: tiles 0..D-1 in flight (fp8 KV: 0..2 in flight, tile 0
  // in LDS), pages of the next ones loaded
  auto page_index = [&](int tt) { return piece_page(a.kv_indices, pc.ip0, pc.nrows, tt * kTileRows + my_row, sh); };
  // LDS ring: the K fragments of the tile in slot `sl`: lane (c16, g) reads
  // chunks 4j + g of row 16w + c16, at kpos(c16, 4j + g).  With a = (c16 >> 2) & 3
  // that position is 4 (j ^ 2 (a & 1)) + (g ^ a) for j < 8 and 32 + (g ^ a)
  // for j = 8, so each chunk's byte offset is one of three per-lane bases plus
  // 64 j: a constant the LDS reads take as an immediate offset.
  [[maybe_unused]] uint32_t k_lo = 0, k_hi = 0, k_v8 = 0;
  if constexpr (kLds) {
    const int ka = (c16 >> 2) & 3;
    const uint32_t kb = (uint32_t)(my_row * kF8Row + 16 * (g ^ ka));
    k_lo = kb + 128u * (ka & 1);  // chunks j with (j & 2) == 0
    k_hi = kb - 128u * (ka & 1);  // chunks j with (j & 2) != 0
    k_v8 = kb + 512u;             // chunk 8 (rope part)
  }
  auto read_k = [&](int sl) {
    if constexpr (kLds) {
      const uint8_t* kslot = &sm.k[sl][0][0];
#pragma unroll
      for (int j = 0; j < L::kChunks; ++j) {
        const uint32_t off = j == 8 ? k_v8 : ((j & 2) ? k_hi : k_lo) + 64u * (j == 8 ? 0 : j);
        kcur[j] = *reinterpret_cast<const u32x4_t*>(kslot + off);
      }
    }
  };
  read_k(0);  // LDS ring: tile 0 is complete since the start's barrier
  // this lane's first 16-byte chunk of its row of tile tt (the row's chunks j are 64 bytes apart)
  auto tile_src = [&](int page, int tt) {
    const int row = page_row(page, pc.nrows, tt * kTileRows + my_row, sh);
    return kvb + (size_t)row * L::kRowBytes + g * 16;
  };

  float m_run[QL];
  float l_run[QL];
  f32x4_t acc[QL][8];
#pragma unroll
  for (int q = 0; q < QL; ++q) {
    m_run[q] = -INFINITY;
    l_run[q] = 0.f;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) acc[q][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // O^T += V^T . P^T over the 64 rows of tile `tt`, this wave's 128 columns,
  // for every token of the pass (the V operands are built once).
  // k-step ks covers rows 32ks..32ks+31; slot s of lane group g is row
  // R = 32ks + (s/4)*16 + g*4 + s%4, which is wave 2ks + s/4's row g*4 + s%4.
  // Block jb holds columns 128w + 16 jb + m (register ring, fp8 KV) or
  // 128w + 8m + jb, m = 0..15; lane c16 feeds m = c16.
  // LDS ring: the next P.V's operands, read from LDS ahead of it (V of the
  // tile, still in its slot, right after the previous P.V; its weights right
  // after the barrier that publishes them), so that the next step's products
  // wait for no LDS read
  [[maybe_unused]] u32x2_t vreg[2][8];
  [[maybe_unused]] u32x2_t preg[QL][2][2];
  // V of tile tt: columns 128w + 8 c16 .. + 7 of row R lie in chunk 8w + c16 / 2,
  // half c16 & 1; these rows have (R >> 2) & 3 == g, so the chunk sits at kpos(4g, 8w + c16 / 2)
  auto load_v = [&](int tt) {
    if constexpr (kLds) {
      const uint8_t* vt = &sm.k[tt & (kSlots - 1)][0][0];
      const int vcol = (kpos(4 * g, 8 * w + (c16 >> 1)) << 4) + ((c16 & 1) << 3);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int R = 32 * ks + (sl >> 2) * 16 + g * 4 + (sl & 3);
          vreg[ks][sl] = *reinterpret_cast<const u32x2_t*>(vt + R * kF8Row + vcol);
        }
    }
  };
  // Register ring, fp8 V: for k-step ks and column block jb (the wave's columns
  // 16 jb .. 16 jb + 15) lane (c16, g) needs column 16 jb + c16 over the rows
  // R(ks, g, s), s < 8, in the P operand's order.  One transposed read gives
  // exactly that when lane (c16, g) addresses row R(ks, g, c16 / 2), columns
  // 16 jb + 8 (c16 & 1) .. + 7.  (In the LDS ring the same reads, through the
  // chunk swizzle, made the launch ~25% slower.)
  [[maybe_unused]] const int v_row = 16 * (c16 >> 3) + 4 * g + ((c16 >> 1) & 3);  // R(0, g, c16 / 2)
  auto load_p = [&](int tt) {
    if constexpr (kLds) {
#pragma unroll
      for (int q = 0; q < QL; ++q)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          preg[q][ks][0] = sm.p[tt & 1][q][2 * ks][lane];
          preg[q][ks][1] = sm.p[tt & 1][q][2 * ks + 1][lane];
        }
    }
  };

  auto pv = [&](int tt) {
    const int buf = tt & 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t pop[QL];
#pragma unroll
      for (int q = 0; q < QL; ++q) {
        u32x4_t pp;
        u32x2_t p0, p1;
        if constexpr (kLds) {
          p0 = preg[q][ks][0];
          p1 = preg[q][ks][1];
        } else {
          p0 = sm.p[buf][q][2 * ks][lane];
          p1 = sm.p[buf][q][2 * ks + 1][lane];
        }
        pp[0] = p0[0];
        pp[1] = p0[1];
        pp[2] = p1[0];
        pp[3] = p1[1];
        pop[q] = __builtin_bit_cast(bf16x8_t, pp);
      }
      if constexpr (KT == Dt::FP8 && !kLds) {
        // column block jb: one transposed read, widened to bf16, one product per token
        u32x2_t rv[8];
        const uint8_t* vb = &sm.v[buf][v_row + 32 * ks][kColsPerWave * w + ((c16 & 1) << 3)];
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) rv[jb] = lds_read_tr8(vb + 16 * jb);
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
          const bf16x8_t op = fp8x8_to_bf16x8(rv[jb][0], rv[jb][1]);
#pragma unroll
          for (int q = 0; q < QL; ++q)
            acc[q][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, pop[q], acc[q][jb], 0, 0, 0);
        }
      } else if constexpr (KT == Dt::FP8) {
        // LDS ring: 8-byte runs of 8 rows (read by load_v), interleaved with
        // v_perm while widening
        u32x2_t rv[8];
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) rv[sl] = vreg[ks][sl];
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
          u32x4_t op[4];
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            const uint32_t A = rv[2 * pr][wd];
            const uint32_t B = rv[2 * pr + 1][wd];
            const uint32_t lo = __builtin_amdgcn_perm(A, B, 0x01050004u);  // A.b0 B.b0 A.b1 B.b1
            const uint32_t hi = __builtin_amdgcn_perm(A, B, 0x03070206u);  // A.b2 B.b2 A.b3 B.b3
            op[0][pr] = fp8x2_to_bf16x2(lo, false);
            op[1][pr] = fp8x2_to_bf16x2(lo, true);
            op[2][pr] = fp8x2_to_bf16x2(hi, false);
            op[3][pr] = fp8x2_to_bf16x2(hi, true);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int jb = wd * 4 + u;
#pragma unroll
            for (int q = 0; q < QL; ++q)
              acc[q][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, op[u]), pop[q],
                                                                   acc[q][jb], 0, 0, 0);
          }
        }
      } else {
        u32x4_t rv[8];
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int R = 32 * ks + (sl >> 2) * 16 + g * 4 + (sl & 3);
          rv[sl] = *reinterpret_cast<const u32x4_t*>(&sm.v[buf][R][(kColsPerWave * w + c16 * 8) * 2]);
        }
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
          const uint32_t sel = (jb & 1) ? 0x03020706u : 0x01000504u;
          u32x4_t op;
#pragma unroll
          for (int pr = 0; pr < 4; ++pr)
            op[pr] = __builtin_amdgcn_perm(rv[2 * pr][jb >> 1], rv[2 * pr + 1][jb >> 1], sel);
#pragma unroll
          for (int q = 0; q < QL; ++q)
            acc[q][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, op), pop[q],
                                                                 acc[q][jb], 0, 0, 0);
        }
      }
    }
  };

  // One tile: `kc` is the ring slot (a compile-time constant), `refill` says
  // whether to start the loads of tile tt + D into the slot just consumed.
  // P.V runs one tile behind S^T, so the MFMA / conversion work of both sits
  // between the same two barriers; the weights of tile tt are made with the
  // running max known before it and kept unless some score of the tile exceeds
  // that max by more than the slack (then every wave rescales and redoes them).
  auto step = [&](auto kc, int tt, auto refill, auto pend_in) {
    constexpr int k = decltype(kc)::value;
    const int buf = tt & 1;
    // ---- S^T for this wave's 16 rows and each token (two accumulation chains); V part to LDS
    f32x4_t s0[QL], s1[QL];
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      s0[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s1[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // LDS ring: the rows of tile tt + 3 (its slot, tile tt - 1's, frees at
    // this step's barrier; its loads go out during the next step's S^T),
    // exchanged now so that the loads need no wait
    [[maybe_unused]] DmaRows next_rows;
    if constexpr (kLds && decltype(refill)::value) {
      constexpr int sl = (k + kSlots - 1) % kSlots;
      next_rows = dma_rows(page_row(ring.first[sl], pc.nrows, (tt + kSlots - 1) * kTileRows + my_row, sh), dl);
    }
    if constexpr (kLds) {
      // K fragments of tile tt: read from its slot right after the barrier
      // that made it complete (the previous step's, or the start's), so the
      // products start at once
      const u32x4_t (&kk)[L::kChunks] = kcur;
      // tile tt + 2's loads (pending since the last barrier) go out one per
      // chunk, between the products: the four waves' 36 loads then reach the
      // address unit spread over the step instead of as one burst after the
      // barrier, which held every wave for ~460 cycles
      uint8_t* pslot = &sm.k[(k + 2) % kSlots][0][0] + wrow_bytes;
#pragma unroll
      for (int j = 0; j < L::kChunks; ++j) {
        if constexpr (decltype(pend_in)::value) {
          __builtin_amdgcn_sched_barrier(0);
          dma_one(a.kv, pslot, pend, dl, j);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (QT == Dt::BF16) {
          // bf16 Q over fp8 K: the fp8 values widen to bf16 exactly
          const bf16x8_t k0 = fp8x8_to_bf16x8(kk[j][0], kk[j][1]);
          const bf16x8_t k1 = fp8x8_to_bf16x8(kk[j][2], kk[j][3]);
#pragma unroll
          for (int q = 0; q < QL; ++q) {
            s0[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb[q][2 * j], s0[q], 0, 0, 0);
            s1[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb[q][2 * j + 1], s1[q], 0, 0, 0);
          }
        } else {
          const uint64_t k0 = (uint64_t)kk[j][0] | ((uint64_t)kk[j][1] << 32);
          const uint64_t k1 = (uint64_t)kk[j][2] | ((uint64_t)kk[j][3] << 32);
#pragma unroll
          for (int q = 0; q < QL; ++q) {
            s0[q] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)k0, (long)q8[q][2 * j], s0[q], 0, 0, 0);
            s1[q] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)k1, (long)q8[q][2 * j + 1], s1[q], 0, 0, 0);
          }
        }
      }
      // the page of the tile this slot receives after tile tt + 2
      if constexpr (decltype(pend_in)::value) ring.first[(k + 2) % kSlots] = page_index(tt + 2 * kSlots - 2);
      // Tile tt + 1's rows of this wave are its own loads, so its K fragments
      // need no barrier, only those loads: after them this wave has issued
      // one page load, then (in this step) tile tt + 2's loads and one page
      // load, kTileOps + 1 in every step that issues a tile (one that issues
      // none waits for everything).  Read now, they arrive while the P.V and
      // the softmax run instead of after the barrier.
      if constexpr (decltype(pend_in)::value)
        wait_vm<kTileOps + 1>();
      else
        wait_vm<0>();
      read_k((k + 1) % kSlots);
    } else {
      auto& dat = ring.dat;
      auto& idxn = ring.next;
      uint8_t* vrow = &sm.v[buf][16 * w + c16][0];
      // The slot is refilled with tile tt + D chunk by chunk, each load issued
      // right after its chunk is used (rows past the piece clamp to its last
      // row, so every steady-state trip issues the same loads and the compiler's
      // wait counts stay exact).  Spread over the products, the four waves' loads
      // reach the address unit a few at a time instead of as one burst.
      // The index of tile tt + 2D goes out before these refills, so the next
      // use of the slot waits for it without waiting for all of its tile.
      const uint8_t* nsrc = nullptr;
      if constexpr (decltype(refill)::value) {
        nsrc = tile_src(idxn[k], tt + D);
        idxn[k] = page_index(tt + 2 * D);
      }
      // bf16 Q over fp8 K: chunk j + 1 is widened while chunk j's products run
      // (the fences around each refill would otherwise keep them apart)
      [[maybe_unused]] bf16x8_t wk0, wk1;
      if constexpr (QT == Dt::BF16 && KT == Dt::FP8) {
        wk0 = fp8x8_to_bf16x8(dat[k][0][0], dat[k][0][1]);
        wk1 = fp8x8_to_bf16x8(dat[k][0][2], dat[k][0][3]);
      }
#pragma unroll
      for (int j = 0; j < L::kChunks; ++j) {
        const u32x4_t kk = dat[k][j];
        if (j < L::kVChunks) *reinterpret_cast<u32x4_t*>(vrow + (j * 4 + g) * 16) = kk;
        if constexpr (KT == Dt::BF16) {
          const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kk);
#pragma unroll
          for (int q = 0; q < QL; ++q) {
            if (j & 1)
              s1[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb[q][j], s1[q], 0, 0, 0);
            else
              s0[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb[q][j], s0[q], 0, 0, 0);
          }
        } else if constexpr (QT == Dt::BF16) {
          const bf16x8_t k0 = wk0;
          const bf16x8_t k1 = wk1;
          if (j + 1 < L::kChunks) {
            wk0 = fp8x8_to_bf16x8(dat[k][j + 1][0], dat[k][j + 1][1]);
            wk1 = fp8x8_to_bf16x8(dat[k][j + 1][2], dat[k][j + 1][3]);
          }
#pragma unroll
          for (int q = 0; q < QL; ++q) {
            s0[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb[q][2 * j], s0[q], 0, 0, 0);
            s1[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb[q][2 * j + 1], s1[q], 0, 0, 0);
          }
        } else {
          const uint64_t k0 = (uint64_t)kk[0] | ((uint64_t)kk[1] << 32);
          const uint64_t k1 = (uint64_t)kk[2] | ((uint64_t)kk[3] << 32);
#pragma unroll
          for (int q = 0; q < QL; ++q) {
            s0[q] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)k0, (long)q8[q][2 * j], s0[q], 0, 0, 0);
            s1[q] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)k1, (long)q8[q][2 * j + 1], s1[q], 0, 0, 0);
          }
        }
        if constexpr (decltype(refill)::value) {
          __builtin_amdgcn_sched_barrier(0);
          dat[k][j] = *reinterpret_cast<const u32x4_t*>(nsrc + j * 64);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // ---- previous tile's P.V (its weights and V were published before the last barrier)
    if (tt > 0) pv(tt - 1);
    // LDS ring: tile tt's V for the next P.V (the tile is whole since the last
    // barrier; its slot is rewritten only after the next one)
    if constexpr (kLds) load_v(tt);
    // ---- scores (log2 domain), masked past the rows each token sees
    float x[QL][4];
    float mx[QL];
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      const f32x4_t sc = s0[q] + s1[q];
      float y[4];
      logit.apply<kCap>(sc, y);
      mx[q] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pr = tt * kTileRows + 16 * w + g * 4 + i;
        x[q][i] = (pr < pc.lim[q]) ? y[i] : -INFINITY;
        mx[q] = fmaxf(mx[q], x[q][i]);
      }
    }
    quad_max<QL>(mx);  // over the wave's 16 rows of each head
#pragma unroll
    for (int q = 0; q < QL; ++q)
      if (g == 0) sm.mx[buf][w][q][c16] = mx[q];
    // ---- speculative weights with the running max known so far
    u32x2_t pw[QL];
    auto make_p = [&]() {
#pragma unroll
      for (int q = 0; q < QL; ++q) {
        float pv4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv4[i] = (x[q][i] == -INFINITY) ? 0.f : fast_exp2(x[q][i] - m_run[q]);
        pw[q][0] = pack_bf16x2(pv4[0], pv4[1]);
        pw[q][1] = pack_bf16x2(pv4[2], pv4[3]);
        sm.p[buf][q][w][lane] = pw[q];
      }
    };
    make_p();
    if constexpr (kLds) {
      // every wave's rows of tile tt + 1 are in LDS (each waited for its own)
      lds_barrier();
      // tile tt - 1's slot is free now (every wave finished its P.V before the
      // barrier): tile tt + 3 goes there, during the next step's S^T
      if constexpr (decltype(refill)::value) pend = next_rows;
    } else {
      __syncthreads();
    }
    // ---- every wave sees the same four maxima, so the decision is workgroup-uniform
    float mxw[QL][kWaves];
#pragma unroll
    for (int q = 0; q < QL; ++q)
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) mxw[q][ww] = sm.mx[buf][ww][q][c16];
    float mt[QL];
    bool need[QL];
    bool any = false;
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      mt[q] = fmaxf(fmaxf(mxw[q][0], mxw[q][1]), fmaxf(mxw[q][2], mxw[q][3]));
      need[q] = mt[q] > m_run[q] + kRescaleSlack;
      any = any || need[q];
    }
    if (__builtin_amdgcn_ballot_w64(any) != 0ull) {
#pragma unroll
      for (int q = 0; q < QL; ++q) {
        const float m_new = need[q] ? mt[q] : m_run[q];
        const float alpha = (m_new == m_run[q]) ? 1.0f : fast_exp2(m_run[q] - m_new);
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) acc[q][jb] *= alpha;
        l_run[q] *= alpha;
        m_run[q] = m_new;
      }
      make_p();  // nobody reads tile tt's weights before the next step
      if constexpr (kLds)
        lds_barrier();
      else
        __syncthreads();
    }
    load_p(tt);  // the weights of tile tt, final now, for the next step's P.V
    // the row sums use the same bf16-rounded weights the P.V product sees
#pragma unroll
    for (int q = 0; q < QL; ++q)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        l_run[q] += __builtin_bit_cast(float, pw[q][i] << 16) + __builtin_bit_cast(float, pw[q][i] & 0xFFFF0000u);
  };

  using Y = std::true_type;
  using N = std::false_type;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  static_assert(D <= 4, "ring depth above 4 needs more unrolled steps");
  if constexpr (kLds) {
    // Whole turns while tiles remain past the turn, then the last 1..4 tiles,
    // whose steps issue only tiles of the piece (when T is a multiple of 4,
    // the usual case, no load past the piece goes out and no step waits for
    // one): 4 left: the first two steps issue the last two tiles; 3 left:
    // the first issues the last; 2 or 1 left: they are in flight already.
    int t0 = 0;
    for (; t0 + 4 < T; t0 += 4) {
      step(S0{}, t0, Y{}, Y{});
      step(S1{}, t0 + 1, Y{}, Y{});
      step(S2{}, t0 + 2, Y{}, Y{});
      step(S3{}, t0 + 3, Y{}, Y{});
    }
    const int r = T - t0;
    if (r == 4) {
      step(S0{}, t0, Y{}, Y{});
      step(S1{}, t0 + 1, N{}, Y{});
    } else if (r == 3) {
      step(S0{}, t0, N{}, Y{});
    } else if (r > 0) {
      step(S0{}, t0, N{}, N{});
    }
    if (r == 2 || r == 3) step(S1{}, t0 + 1, N{}, N{});
    if (r >= 3) step(S2{}, t0 + 2, N{}, N{});
    if (r == 4) step(S3{}, t0 + 3, N{}, N{});
  } else {
    int t0 = 0;
    for (; t0 + D <= T; t0 += D) {
      step(S0{}, t0, Y{}, N{});
      if constexpr (D > 1) step(S1{}, t0 + 1, Y{}, N{});
      if constexpr (D > 2) step(S2{}, t0 + 2, Y{}, N{});
      if constexpr (D > 3) step(S3{}, t0 + 3, Y{}, N{});
    }
    // the last T mod D tiles are already in the ring
    if (t0 < T) step(S0{}, t0, N{}, N{});
    if constexpr (D > 1)
      if (t0 + 1 < T) step(S1{}, t0 + 1, N{}, N{});
    if constexpr (D > 2)
      if (t0 + 2 < T) step(S2{}, t0 + 2, N{}, N{});
  }
  if (T > 0) pv(T - 1);

  // ---- finish: per-head row sums of the 4 waves, then this wave's 128 columns
#pragma unroll
  for (int q = 0; q < QL; ++q) {
    const float l_tot = pair_sum32(pair_sum16(l_run[q]));
    if (g == 0) sm.lsum[w][q][c16] = l_tot;
  }
  if constexpr (kLds) wait_vm<0>();  // no tile load may still land in the staging slot
  __syncthreads();
  // Lane (c16, g) holds, for block jb and i < 4, head c16 at column
  // 128w + 16 jb + 4g + i (register ring, fp8 KV: four neighbouring columns
  // per block) or 128w + (4g+i)*8 + jb (a contiguous run of 32 columns).  With one
  // token per pass each wave stages its rows in LDS (the V buffers are free
  // once the last P.V is done) and reads them back so that every store covers
  // whole runs of the wave's 128 columns of 2 heads (float32) or 4 heads
  // (bf16); reads follow the same wave's writes in issue order.  Two-token
  // passes of fp8 Q stage one token after the other; those of bf16 Q store
  // straight from the registers.
  uint8_t* const stage = sm.out_stage() + (size_t)w * kOutStageBytes;
#pragma unroll
  for (int q = 0; q < QL; ++q) {
    if (q >= pc.ntok) break;  // uniform
    const float Lsum = sm.lsum[0][q][c16] + sm.lsum[1][q][c16] + sm.lsum[2][q][c16] + sm.lsum[3][q][c16];
    const float scale = Lsum > 0.f ? out_mul / Lsum : 0.f;
    const int t = pc.t0 + q;
    if constexpr (QL > 1 && QT == Dt::BF16 && KT == Dt::FP8) {
      // two tokens of bf16 Q: stored straight from the registers (staging
      // them spilled)
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        const int col = kColsPerWave * w + 16 * jb + 4 * g;
        if (pc.complete) {
          const u32x2_t pk{pack_bf16x2(acc[q][jb][0] * scale, acc[q][jb][1] * scale),
                           pack_bf16x2(acc[q][jb][2] * scale, acc[q][jb][3] * scale)};
          *reinterpret_cast<u32x2_t*>(a.out + ((size_t)t * kHeads + c16) * kVDim + col) = pk;
        } else {
          *reinterpret_cast<f32x4_t*>(a.part_o + ((size_t)(pc.slot + q) * kHeads + c16) * kVDim + col) =
              acc[q][jb] * scale;
        }
      }
    } else if constexpr (QL > 1 && KT == Dt::FP8) {
      // staged like one token, token by token (each wave reuses its area once
      // its own reads of the previous token are done: LDS operations of one
      // wave complete in order)
      if (pc.complete) {
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
          const u32x2_t pk{pack_bf16x2(acc[q][jb][0] * scale, acc[q][jb][1] * scale),
                           pack_bf16x2(acc[q][jb][2] * scale, acc[q][jb][3] * scale)};
          *reinterpret_cast<u32x2_t*>(stage + c16 * kOutPitchBf16 + (16 * jb + 4 * g) * 2) = pk;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r = 0; r < kHeads / 4; ++r) {
          const int h = 4 * r + (lane >> 4);
          const int c = lane & 15;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + h * kOutPitchBf16 + c * 16);
          st_stream(v, a.out + ((size_t)t * kHeads + h) * kVDim + kColsPerWave * w + c * 8);
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
          *reinterpret_cast<f32x4_t*>(stage + c16 * kOutPitchF32 + (16 * jb + 4 * g) * 4) = acc[q][jb] * scale;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r = 0; r < kHeads / 2; ++r) {
          const int h = 2 * r + (lane >> 5);
          const int c = lane & 31;
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage + h * kOutPitchF32 + c * 16);
          st_stream(v, a.part_o + ((size_t)(pc.slot + q) * kHeads + h) * kVDim + kColsPerWave * w + c * 4);
        }
      }
      __builtin_amdgcn_wave_barrier();
    } else if (pc.complete) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4_t pk;
#pragma unroll
        for (int u = 0; u < 4; ++u) pk[u] = pack_bf16x2(acc[q][2 * u][i] * scale, acc[q][2 * u + 1][i] * scale);
        *reinterpret_cast<u32x4_t*>(stage + c16 * kOutPitchBf16 + (4 * g + i) * 16) = pk;
      }
      __builtin_amdgcn_wave_barrier();
      // The last pass of a workgroup streams its rows out (non-temporal: no
      // line stays dirty in the L2 for the write-back at the launch's end).
      // A pass that another follows stores them plainly: the next pass's first
      // waits count these stores too (the vector-memory count covers loads and
      // stores in issue order), and a plain store completes in the L2, a
      // streamed one only in memory.  The empty asm statements keep the
      // compiler from folding the two loops into one, which drops the hint.
      if (pc.last) {
#pragma unroll
        for (int r = 0; r < kHeads / 4; ++r) {
          const int h = 4 * r + (lane >> 4);
          const int c = lane & 15;  // 16-byte piece of the head's 256 bytes
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + h * kOutPitchBf16 + c * 16);
          st_stream(v, a.out + ((size_t)t * kHeads + h) * kVDim + kColsPerWave * w + c * 8);
        }
      } else {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < kHeads / 4; ++r) {
          const int h = 4 * r + (lane >> 4);
          const int c = lane & 15;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + h * kOutPitchBf16 + c * 16);
          *reinterpret_cast<u32x4_t*>(a.out + ((size_t)t * kHeads + h) * kVDim + kColsPerWave * w + c * 8) = v;
        }
        asm volatile("" ::: "memory");
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4_t v0, v1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v0[u] = acc[q][u][i] * scale;
          v1[u] = acc[q][4 + u][i] * scale;
        }
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(stage + c16 * kOutPitchF32 + (4 * g + i) * 32);
        dst[0] = v0;
        dst[1] = v1;
      }
      __builtin_amdgcn_wave_barrier();
      if (pc.last) {  // streamed or plain, as for the bf16 rows above
#pragma unroll
        for (int r = 0; r < kHeads / 2; ++r) {
          const int h = 2 * r + (lane >> 5);
          const int c = lane & 31;  // 16-byte piece of the head's 512 bytes
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage + h * kOutPitchF32 + c * 16);
          st_stream(v, a.part_o + ((size_t)(pc.slot + q) * kHeads + h) * kVDim + kColsPerWave * w + c * 4);
        }
      } else {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < kHeads / 2; ++r) {
          const int h = 2 * r + (lane >> 5);
          const int c = lane & 31;
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage + h * kOutPitchF32 + c * 16);
          *reinterpret_cast<f32x4_t*>(a.part_o + ((size_t)(pc.slot + q) * kHeads + h) * kVDim + kColsPerWave * w +
                                      c * 4) = v;
        }
        asm volatile("" ::: "memory");
      }
    }
    if constexpr (QL > 1 && KT == Dt::BF16) __builtin_amdgcn_wave_barrier();  // the next token reuses the area
    if (w == 0 && g == 0) {
      // no visible row: -inf (no weight in a merge); a NaN sum (NaN inputs) stays NaN so that it
      // propagates through the merge as it does through an unsplit sequence
      const float lse2 = Lsum == 0.f ? -INFINITY : m_run[q] + fast_log2(Lsum);
      if (!pc.complete)
        __builtin_nontemporal_store(lse2, &a.part_lse[(pc.slot + q) * kHeads + c16]);
      else if (a.lse_out != nullptr)
        a.lse_out[(size_t)t * kHeads + c16] = lse2 * kLn2;
    }
  }
  __syncthreads();  // the shared tile and sums may be reused by the next piece
}

// ------------------------------------------------------------------ kernels

// Query tokens and last-page rows of one sequence, packed (tokens << 16) | rows.
// With one token per sequence at most, qo_e is not read.
__device__ __forceinline__ int pack_seq_aux(const Args& a, int qo_b, int qo_e, int last_raw, bool paged) {
  const int ql = a.max_q_len > 1 ? min(max(qo_e - qo_b, 0), a.max_q_len) : 1;
  const int last = paged ? min(max(last_raw, 1), 1 << a.page_shift) : 1 << a.page_shift;
  return (ql << 16) | last;
}

// kForm 0: the plain decode (pages of one row, one token, no cap); 1: the
// general form without the soft-cap; 2: the general form with it.
template <Dt QT, Dt KT, bool kBigBatch, int QL, int kForm>
__global__ __launch_bounds__(kThreads) void mla_decode_kernel(Args a) {
  static_assert(kForm >= 0 && kForm <= 2, "three kernel forms");
  constexpr bool kGeneral = kForm > 0;
  constexpr bool kCap = kForm == 2;
  static_assert(kGeneral || QL == 1, "several tokens per walk only in the general form");
  __shared__ Smem<KT, QL> sm;
  constexpr int kScanPerThread = scan_per_thread<KT, QL>();
  constexpr int kSeqTable = seq_table<KT, QL>();
  const int sh = kGeneral ? a.page_shift : 0;
  const bool paged = a.kv_last_page_len != nullptr && sh > 0;
  const bool multi = a.max_q_len > 1;  // several tokens per sequence: read qo_indptr[b + 1] too
  // First round trip: the split geometry and the indptr values of up to
  // kScanPerThread sequences per thread (everything the start needs, so no
  // later load has to wait behind the ring's loads: waits count in order).
  // The loads are unconditional (index clamped into the batch, an unpaged
  // call reads kv_indptr in place of the last-page lengths) and only the raw
  // values are kept: a branch around a load, or using its value here, would
  // make each load wait for the previous ones.
  const int32_t* last_src = paged ? a.kv_last_page_len : a.kv_indptr;
  int sv[kScanPerThread][5];
#pragma unroll
  for (int i = 0; i < kScanPerThread; ++i) {
    const int j = min((int)threadIdx.x + i * kThreads, a.batch - 1);
    sv[i][0] = a.kv_indptr[j];
    sv[i][1] = a.kv_indptr[j + 1];
    sv[i][2] = a.qo_indptr[j];
    sv[i][3] = a.qo_indptr[j + 1];
    sv[i][4] = last_src[j];
  }
  const float qs = (QT == Dt::FP8) ? *a.q_scale : 1.0f;
  const float ks = (KT == Dt::FP8) ? *a.kv_scale : 1.0f;
  // the ends of the row space, for the cost-free split: loaded here, in the
  // same round trip, because a load placed where the split is computed would
  // go out only after the table's values have arrived (a second round trip
  // before the ring's indices can be requested)
  const int32_t ip_first = a.kv_indptr[0];
  const int32_t ip_last = a.kv_indptr[a.batch];
  // The two float arguments are first used after the start's barriers; read
  // there, their scalar load (and its wait) went out only then, on the path
  // to the first tile.  Read now, it overlaps the first round trip.
  const float sm_scale = a.sm_scale;
  const float logit_cap = a.logit_cap;
  asm volatile("" ::"s"(sm_scale), "s"(logit_cap));
  // these loads go out before the ring's, so using them never waits for the ring's indices
  __builtin_amdgcn_sched_barrier(0);
  // LDS ring: the per-lane constants of the tile loads, computed while the
  // first round trip is in flight (an empty asm use keeps the compiler from
  // sinking their ~100 instructions to the first piece, after the barriers,
  // where they would delay its first tile)
  [[maybe_unused]] DmaLanes dl;
  if constexpr (lds_ring<KT, QL>()) {
    dl = dma_lanes();
#pragma unroll
    for (int i = 0; i < 9; ++i) asm volatile("" ::"v"(dl.src[i]), "v"(dl.off[i]));
  }

  // The first round trip's values go to the LDS sequence table before the
  // ring's indices are requested, so no register waiting on them stays live
  // while the indices are in flight (the compiler's wait counts would
  // otherwise drain the indices at the first join).  The same pass finds
  // whether every sequence is as long as the first, which the split needs (a
  // ballot per wave, so no shuffle chain).
  // Every entry is written, past the batch too (with the clamped values;
  // nothing reads those): a load consumed on one path only would make the
  // compiler wait for all loads, the ring's included, where the paths join.
  const int len0 = a.kv_indptr[1] - a.kv_indptr[0];
  bool differs = false;
#pragma unroll
  for (int i = 0; i < kScanPerThread; ++i) {
    const int j = threadIdx.x + i * kThreads;
    sm.seq[j][0] = sv[i][0];
    sm.seq[j][1] = sv[i][1];
    sm.seq[j][2] = sv[i][2];
    sm.seq[j][3] = pack_seq_aux(a, sv[i][2], sv[i][3], sv[i][4], paged);
    differs |= (j < a.batch) & (sv[i][1] - sv[i][0] != len0);
  }
  if constexpr (kBigBatch) {
    for (int j = threadIdx.x + kSeqTable; j < a.batch; j += kThreads)
      differs |= a.kv_indptr[j + 1] - a.kv_indptr[j] != len0;
  }
  const bool wave_differs = __ballot(differs) != 0;
  if ((threadIdx.x & 63) == 0) sm.differs[threadIdx.x >> 6] = wave_differs ? 1 : 0;
  if (threadIdx.x == 0) {
    sm.bmin = 0x7fffffff;
    sm.bmax = -1;
  }

  // The split is known only after the barrier below, but the cost-free one
  // (the usual one for uniform lengths) is known now, and under it the first
  // piece always starts at the share start (the sequence holding position lo
  // begins at or before it).  So the page indices of that piece's ring are
  // fetched now, clamped to the share's pages, while the barrier and the scan
  // below run; the piece issues the rows once its Q is on the way.  If the
  // split turns out to carry the cost, the pieces fetch their own.
  const int k = blockIdx.x;
  RingOf<QT, KT, QL> ring;
  const Geo g0 = cost_free_geo(ip_first, ip_last, a.units, a.min_chunk, sh);
  {
    const int lo0 = k * g0.chunk;
    if (lo0 < g0.total) {  // a share with positions: its indices exist
      issue_ring_indices(a.kv_indices, g0.base + lo0, (min(lo0 + g0.chunk, g0.total) - lo0) << sh, sh, ring);
    }
  }
  __syncthreads();  // the table, the length flags and bmin / bmax are in place
  const bool uniform = (sm.differs[0] | sm.differs[1] | sm.differs[2] | sm.differs[3]) == 0;
  const Geo geo = make_geo(g0, a.batch, a.units, a.min_chunk, sh, uniform ? len0 : -1);
  if (k >= geo.n_wg) return;
  if (k == 0 && threadIdx.x < 5) {  // the split, for the merge launch
    const int32_t v[5] = {geo.base, geo.cost, geo.total, geo.chunk, geo.n_wg};
    a.counters[a.batch + threadIdx.x] = v[threadIdx.x];
  }
  const int lo = k * geo.chunk;
  const int hi = min(lo + geo.chunk, geo.total);

  const float c_nat = sm_scale * qs * ks;
  Logit logit;
  logit.c_score = c_nat * kLog2e;
  logit.k1 = kCap ? 2.0f * kLog2e * c_nat / logit_cap : 0.f;
  logit.k2 = logit_cap * kLog2e;
  const float out_mul = ks;

  const bool primed = geo.cost == 0;  // the ring's indices above are the first piece's
  // (empty sequences are zeroed after the pieces: stores here would enter the
  // compiler's count of loads in flight and make the prologue wait for all)
  auto scan_one = [&](int j, int ipb, int ipe) {
    const int st = ipb - geo.base + geo.cost * j;
    const int en = st + (ipe - ipb);
    if (en > st && st < hi && en > lo) {
      atomicMin(&sm.bmin, j);
      atomicMax(&sm.bmax, j);
    }
  };
#pragma unroll
  for (int i = 0; i < kScanPerThread; ++i) {
    const int j = threadIdx.x + i * kThreads;
    if (j < a.batch) scan_one(j, sm.seq[j][0], sm.seq[j][1]);
  }
  // Sequences past the LDS table (only in the big-batch instantiation: a loop
  // that merely never runs would still make the compiler drain every load
  // in flight, the ring's indices included, where its branch rejoins).
  if constexpr (kBigBatch) {
    for (int j = threadIdx.x + kSeqTable; j < a.batch; j += kThreads) scan_one(j, a.kv_indptr[j], a.kv_indptr[j + 1]);
  }
  __syncthreads();
  const int bmin = sm.bmin;
  const int bmax = sm.bmax;

  for (int b = bmin; b <= bmax; ++b) {
    // From the LDS table (batches up to kSeqTable), else from memory.  Two
    // instantiations rather than a runtime select: a select between the two
    // addresses becomes a generic load, whose wait would drain the ring.
    int ipb, ipe, t, aux;
    if constexpr (!kBigBatch) {
      ipb = sm.seq[b][0];
      ipe = sm.seq[b][1];
      t = sm.seq[b][2];
      aux = sm.seq[b][3];
    } else {
      ipb = a.kv_indptr[b];
      ipe = a.kv_indptr[b + 1];
      t = a.qo_indptr[b];
      aux = pack_seq_aux(a, t, multi ? a.qo_indptr[b + 1] : 0, paged ? a.kv_last_page_len[b] : 0, paged);
    }
    const int st = ipb - geo.base + geo.cost * b;  // the sequence's positions in the split space
    const int en = st + (ipe - ipb);
    if (en <= st) continue;
    const int q_len = aux >> 16;
    const int n_rows = ((en - st - 1) << sh) + (aux & 0xFFFF);  // the last page may be part-filled
    const int s_lo = max(st, lo);
    const int s_hi = min(en, hi);
    const bool complete = (st >= lo) && (en <= hi);
    // this workgroup holds piece k - st / chunk of the sequence
    const int slot = complete ? -1 : part_slot(b, k - st / geo.chunk, st, geo.chunk, a.spec, a.batch);
    const int r0 = (s_lo - st) << sh;  // the piece's first row within the sequence
    const int nrows = min((s_hi - st) << sh, n_rows) - r0;
    for (int tau0 = 0; tau0 < q_len; tau0 += QL) {
      Piece<QL> pc;
      pc.ip0 = ipb + (s_lo - st);
      pc.nrows = nrows;
      pc.t0 = t + tau0;
      pc.ntok = min(QL, q_len - tau0);
#pragma unroll
      for (int q = 0; q < QL; ++q) {
        // causal: token tau of q_len sees the sequence's first n_rows - q_len + 1 + tau rows
        const int vis = a.causal ? n_rows - q_len + 1 + tau0 + q : n_rows;
        pc.lim[q] = (q < pc.ntok) ? min(nrows, vis - r0) : 0;
      }
      pc.slot = complete ? -1 : slot * a.max_q_len + tau0;
      pc.complete = complete;
      pc.last = b == bmax && tau0 + QL >= q_len;
      if (!primed || b != bmin || tau0 != 0) issue_ring_indices(a.kv_indices, pc.ip0, nrows, sh, ring);
      attend_piece<QT, KT, QL, kGeneral, kCap>(a, sm, pc, logit, out_mul, ring, dl);
    }
    if (!complete && a.fused && q_len > 0) {
      __threadfence();
      __syncthreads();
      if (threadIdx.x == 0) sm.arrive = atomicAdd(&a.counters[b], 1);
      __syncthreads();
      const int S = piece_count(st, en, geo.chunk);
      if (sm.arrive == S - 1) {
        __threadfence();
        const int chunk = geo.chunk;
        const int qmax = a.max_q_len;
        const int spec = a.spec;
        const int batch = a.batch;
        const int w = threadIdx.x >> 6;
        for (int tau = 0; tau < q_len; ++tau)
          for (int hh = 0; hh < kHeads / kWaves; ++hh) {
            const int h = w * (kHeads / kWaves) + hh;
            merge_head_wave(
                a.part_o, a.part_lse, S,
                [=](int i) { return part_slot(b, i, st, chunk, spec, batch) * qmax + tau; }, 1.0f, h,
                a.out + ((size_t)(t + tau) * kHeads + h) * kVDim,
                a.lse_out != nullptr ? a.lse_out + (size_t)(t + tau) * kHeads + h : nullptr);
          }
        if (threadIdx.x == 0) atomicExch(&a.counters[b], 0);
      }
      __syncthreads();
    }
  }

  // Empty sequences: zeros, written by the share holding their position.
  for (int j = threadIdx.x; j < a.batch; j += kThreads) {
    int ipb, ipe, qo, aux;
    if constexpr (!kBigBatch) {
      ipb = sm.seq[j][0];
      ipe = sm.seq[j][1];
      qo = sm.seq[j][2];
      aux = sm.seq[j][3];
    } else {
      ipb = a.kv_indptr[j];
      ipe = a.kv_indptr[j + 1];
      qo = a.qo_indptr[j];
      aux = pack_seq_aux(a, qo, multi ? a.qo_indptr[j + 1] : 0, paged ? a.kv_last_page_len[j] : 0, paged);
    }
    if (ipe > ipb) continue;
    int owner = (ipb - geo.base + geo.cost * j) / geo.chunk;
    if (owner > geo.n_wg - 1) owner = geo.n_wg - 1;
    if (owner == k)
      for (int r = 0; r < (aux >> 16); ++r) {
        zero_row_by_thread(a.out + (size_t)(qo + r) * kHeads * kVDim);
        if (a.lse_out != nullptr)
          for (int h = 0; h < kHeads; ++h) a.lse_out[(size_t)(qo + r) * kHeads + h] = -INFINITY;
      }
  }
}

// Separate merge launch: one wave per (sequence, head, token); sequences that
// were not split were finished by the attention kernel and are skipped.
// The arguments the first round trip needs come first, as scalars: the
// library is built to have the command processor preload leading kernel
// arguments into scalar registers, so those loads go out without waiting for
// the kernel-argument segment (the Args copy serves the rest).
__global__ __launch_bounds__(64) void mla_merge_split_kernel(const int32_t* __restrict__ rec,
                                                             const int32_t* __restrict__ kv_indptr,
                                                             const int32_t* __restrict__ qo_indptr,
                                                             const float* __restrict__ part_o,
                                                             const float* __restrict__ part_lse, int32_t spec,
                                                             int32_t qmax, int32_t units, int32_t batch, Args a) {
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int tau = blockIdx.z;
  const int lane = threadIdx.x & 63;
  // The sequence's first `spec` pieces have slots that depend on b alone
  // (part_slot): their loads go out with the first round trip below, before
  // the split is known.  Slots past the sequence's pieces hold stale values
  // and are never used.
  MergePre pre;
  auto pre_load = [&](int u) {
    if (u < spec) {
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(
          part_o + ((size_t)((b * spec + u) * qmax + tau) * kHeads + h) * kVDim + lane * 8);
      pre.a[u] = src[0];
      pre.b[u] = src[1];
    } else {
      pre.a[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pre.b[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
#pragma unroll
  for (int u = 0; u < kMaxSpec / 2; ++u) pre_load(u);
  if (spec > kMaxSpec / 2) {
#pragma unroll
    for (int u = kMaxSpec / 2; u < kMaxSpec; ++u) pre_load(u);
  }
  pre.lse = lane < spec ? part_lse[((b * spec + lane) * qmax + tau) * kHeads + h] : -INFINITY;
  // Every index this wave needs is loaded in the same round trip: a load
  // written after one of the early exits below is issued only once the values
  // that decide the exit have arrived.
  const int32_t* gr = rec;  // the split the attention launch used (after the arrival counters)
  Geo geo;
  geo.base = gr[0];
  geo.cost = gr[1];
  geo.total = gr[2];
  geo.chunk = gr[3];
  geo.n_wg = gr[4];
  const int ipb = kv_indptr[b];
  const int ipe = kv_indptr[b + 1];
  const int qo = qo_indptr[b];
  const int qo_e = qo_indptr[b + 1];
  const int st = ipb - geo.base + geo.cost * b;
  const int en = st + (ipe - ipb);
  const int q_len = qmax > 1 ? min(max(qo_e - qo, 0), qmax) : 1;
  // A split that does not hold this sequence (none recorded yet: chunk 0, or
  // another kv_indptr) is skipped: every slot read below is then below
  // batch * spec + 2 * n_wg <= batch * spec + 2 * units, inside the partial
  // buffers.
  if (en <= st || tau >= q_len) return;
  if (geo.chunk < 1 || geo.n_wg > units || st < 0 || en > geo.total || (en - 1) / geo.chunk >= geo.n_wg) return;
  const int S = piece_count(st, en, geo.chunk);
  if (S <= 1) return;
  uint16_t* const out_head = a.out + ((size_t)(qo + tau) * kHeads + h) * kVDim;
  float* const lse_dst = a.lse_out != nullptr ? a.lse_out + (size_t)(qo + tau) * kHeads + h : nullptr;
  if (S <= spec) {  // every piece is in
    merge_head_wave<true>(part_o, part_lse, S, [](int) { return 0; }, 1.0f, h, out_head, lse_dst, &pre);
  } else {
    const int chunk = geo.chunk;
    merge_head_wave(
        part_o, part_lse, S, [=](int i) { return part_slot(b, i, st, chunk, spec, batch) * qmax + tau; }, 1.0f,
        h, out_head, lse_dst);
  }
}

// Merge of caller-provided partials (natural-log lse), one wave per (sequence, head).
__global__ __launch_bounds__(64) void mla_reduce_external_kernel(const float* part_o, const float* part_lse,
                                                                 const int32_t* part_indptr, uint16_t* out,
                                                                 float* lse_out) {
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int p0 = part_indptr[b];
  const int S = part_indptr[b + 1] - p0;
  // S <= 0 leaves all weights zero and writes zeros
  merge_head_wave(part_o, part_lse, S < 0 ? 0 : S, [=](int i) { return p0 + i; }, kLog2e, h,
                  out + ((size_t)b * kHeads + h) * kVDim, lse_out != nullptr ? lse_out + (size_t)b * kHeads + h : nullptr);
}

// Streaming read probe (a diagnostic): one pass, no loop.  Workgroup k of 512
// threads reads the 2048 sixteen-byte words [2048 k, 2048 k + 2048), four
// loads per thread, all issued before any is used, with the non-temporal hint
// (of the plain read forms measured on this device, one-shot workgroups of
// 512 threads x 4 non-temporal loads read a few hundred MB fastest).  Loads
// past the end read the last word and are then dropped, so every load is
// unconditional.  Each workgroup stores the xor of what it read so that no
// load can be dropped.
constexpr int kProbeThreads = 512;
constexpr int kProbeLoads = 4;
constexpr int kProbeWords = kProbeThreads * kProbeLoads;
__global__ __launch_bounds__(kProbeThreads) void mla_read_probe_kernel(const u32x4_t* __restrict__ p, int64_t n16,
                                                                       uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kProbeThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kProbeWords + threadIdx.x;
  u32x4_t v[kProbeLoads];
#pragma unroll
  for (int u = 0; u < kProbeLoads; ++u) {
    const int64_t i = base + (int64_t)u * kProbeThreads;
    v[u] = __builtin_nontemporal_load(p + (i < n16 ? i : n16 - 1));
  }
  uint32_t x = 0u;
#pragma unroll
  for (int u = 0; u < kProbeLoads; ++u)
    if (base + (int64_t)u * kProbeThreads < n16) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0u;
#pragma unroll
    for (int i = 0; i < kProbeThreads / 64; ++i) r ^= red[i];
    sink[blockIdx.x] = r;
  }
}

__global__ void mla_fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------ step a0: Q cast

// Step a0: groups of eight through the same conversion the attention kernel
// uses for a bf16-supplied fp8 Q (so the exhaustive test of this kernel
// covers both); unaligned heads and tails go value by value.
__global__ void mla_quantize_q_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < n; i += stride) {
    if (i + 8 <= n && ((reinterpret_cast<uintptr_t>(src + i) & 15u) == 0) && ((reinterpret_cast<uintptr_t>(dst + i) & 7u) == 0)) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + i);
      *reinterpret_cast<uint64_t*>(dst + i) = bf16x8_to_e4m3fn(v);
    } else {
      for (int64_t j = i; j < n && j < i + 8; ++j) dst[j] = (uint8_t)bf16_to_e4m3fn(src[j]);
    }
  }
}

// ------------------------------------------- step a0, amax-scaled variant

// float32 -> e4m3fn, round to nearest even, non-saturating (the conventions
// of bf16_to_e4m3fn), on the bit fields.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(uint32_t x) {
  const uint32_t sign = (x >> 24) & 0x80u;
  const int e = (int)((x >> 23) & 0xFFu);
  const uint32_t m = x & 0x7FFFFFu;
  if (e == 0xFF) return sign | 0x7Fu;
  int E = e - 127 + 7;  // e4m3 biased exponent
  if (E >= 1) {
    uint32_t m3 = m >> 20;
    const uint32_t rem = m & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) {
      m3 = 0;
      ++E;
    }
    if (E > 15 || (E == 15 && m3 == 7u)) return sign | 0x7Fu;
    return sign | ((uint32_t)E << 3) | m3;
  }
  // below 2^-6: units of 2^-9; the 24-bit significand is scaled by 2^(e - 141)
  const int shift = 141 - e;
  if (e == 0 || shift > 24) return sign;  // below 2^-10 rounds to zero (2^-10 itself is a tie to even 0)
  const uint32_t sig = 0x800000u | m;
  uint32_t n = sig >> shift;
  const uint32_t rem = sig & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (n & 1u))) ++n;
  return sign | n;  // n == 8 is the smallest normal, encoded the same way
}

// |x| of a finite bf16 as ordered bits (0 for +-inf and NaN, which do not enter the amax).
__device__ __forceinline__ uint32_t finite_abs_bits(uint32_t h) {
  const uint32_t a = h & 0x7FFFu;
  return a < 0x7F80u ? a : 0u;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = max(max(red[0], red[1]), max(red[2], red[3]));
  __syncthreads();
  return v;
}

// Pass 1: each workgroup's amax over its grid-stride share, as ordered bits.
__global__ __launch_bounds__(256) void mla_q_amax_kernel(const uint16_t* __restrict__ src, int64_t n,
                                                         uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
    const int64_t groups = n / 8;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < groups; i += stride) {
      const u32x4_t v = reinterpret_cast<const u32x4_t*>(src)[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) m = max(m, max(finite_abs_bits(v[k] & 0xFFFFu), finite_abs_bits(v[k] >> 16)));
    }
    for (int64_t i = groups * 8 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
      m = max(m, finite_abs_bits(src[i]));
  } else {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) m = max(m, finite_abs_bits(src[i]));
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Pass 2: every workgroup reduces the nparts (<= 256) partial maxima,
// q_scale = amax / 448 in float32 (1 when amax is 0), and casts its share of
// q / q_scale (float32 division, correctly rounded) to e4m3fn; +-inf and NaN
// inputs give the NaN code with their sign.  Workgroup 0 stores q_scale.
__global__ __launch_bounds__(256) void mla_q_cast_scaled_kernel(const uint16_t* __restrict__ src,
                                                                uint8_t* __restrict__ dst, int64_t n,
                                                                const uint32_t* __restrict__ partial, int nparts,
                                                                float* __restrict__ q_scale) {
  __shared__ uint32_t red[4];
  const uint32_t m = block_max_u32(threadIdx.x < (unsigned)nparts ? partial[threadIdx.x] : 0u, red);
  const float amax = __builtin_bit_cast(float, m << 16);
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *q_scale = scale;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const uint32_t h = src[i];
    uint32_t code;
    if ((h & 0x7FFFu) >= 0x7F80u) {
      code = ((h >> 8) & 0x80u) | 0x7Fu;
    } else {
      const float y = __builtin_bit_cast(float, h << 16) / scale;
      code = f32_to_e4m3fn(__builtin_bit_cast(uint32_t, y));
    }
    dst[i] = (uint8_t)code;
  }
}

}  // namespace mla
