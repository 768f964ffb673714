// BigBird block-sparse self-attention forward for MI355X (gfx950, CDNA4).
//
// What is computed (page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
// section "BigBird：从二次方注意力到线性稀疏注意力"; paper card "Big Bird:
// Transformers for Longer Sequences", section "方法适配"):
//   Q/K/V are cut into blocks of BS tokens.  Query blocks 0 and nb-1 attend
//   every key; a middle block i attends blocks {i-1, i, i+1}, {0, nb-1} and
//   its r random blocks.  Logits q.k/sqrt(d), -10000 added on padded keys,
//   one softmax per query row, times V.
//
// How it is laid out on the GPU.  Every workgroup runs one "work unit": one
// query block of one (batch, head) against a short list of key tiles.
//   - middle unit: query block i, tiles [0, band \ globals, nb-1, random...]
//     (5 + r tiles, 4 + r at i = 1 and i = nb-2), finalised in place;
//   - global unit: query block 0 or nb-1 against a chunk of kChunkTiles
//     consecutive key tiles (split-K over L); it writes an unnormalised
//     partial (row max, row sum, O) to the workspace.  A small merge kernel,
//     launched next on the same stream, combines the partials of each global
//     block in fixed chunk order (deterministic).
// The paper packs the attended blocks into dense tensors (rolled key copies,
// gathered random blocks) for TPU matrix units; here each attended block is
// one contiguous BS x 64 slab of K and of V that a workgroup copies from HBM
// into LDS with 16-byte coalesced loads, driven by the random-block table --
// the accelerator point the paper card makes in section "瓶颈" (regular,
// coalesced memory traffic and dense tile products) without any packing.
//
// Inside a workgroup: BS/32 query groups x 2 key halves = one wave each.
// A wave owns 32 query rows and, per key tile, BS/2 keys in 32-key subtiles:
//   S^T(32 keys x 32 queries) = K . Q^T      bf16 MFMA 32x32x16, fp32 acc
//   online softmax in fp32 (lane = one query row, 16 keys per lane)
//   O^T(64 dims x 32 queries) += V^T . P^T   bf16 MFMA 32x32x16
// Computing the transposed products puts one query row in each lane, so the
// row max and sum need one cross-lane step per subtile, and the fp32 score
// registers turn into the PV operand without any data movement: the K rows
// fed to the score MFMA are permuted (perm_row) so that each lane's 16 score
// registers are 2 runs of 8 consecutive keys, exactly the operand layout the
// PV MFMA wants.  V stays row-major in LDS; a transposing LDS read
// (ds_read_b64_tr_b16) hands it to the PV MFMA as V^T.
// The two key-half waves of a query group merge their (max, sum, O) states
// through LDS at the end.
//
// fp32 inputs run the same code with fp32 MFMA (32x32x2) and fp32 P.
//
// Two more forms of the unit kernel share the work units, tile lists,
// partials and merge: bf16 at block 128 runs the 32-key-step kernel (two
// waves of complete rows per workgroup, no merge between waves; its section
// below), and problems with too few units to fill the device run "kind 3"
// units, every query block split over its key tiles (small_split()).  The bf16
// softmax takes a unit's probabilities against one fixed reference per row
// with an exact slow path (softmax_pv(), redo_unit_w()).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "bb_attn.h"

namespace {

constexpr int kD = 64;                   // supported head dimension
constexpr int kChunkTiles = 8;           // key tiles per global-row work unit
constexpr float kScaleLog2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
constexpr float kMaskRaw = -10000.0f * 8.0f;  // -10000 on the logit, in q.k units
constexpr float kRescaleTau = 8.0f;      // lazy rescale threshold (log2 units)
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <typename T, int BS>
struct Cfg {
  static constexpr int ES = sizeof(T);
  static constexpr int ROWB = kD * ES;              // bytes per K/V row
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int QROWS = 64;                  // query rows per work unit
  static constexpr int QSPLIT = BS / QROWS;         // work units per query block (1 or 2)
  static constexpr int WQ = QROWS / 32;             // query groups (32 rows each)
  static constexpr int WK = BS / 32;                // key groups: one 32-key subtile per wave
  static constexpr int NW = WQ * WK;                // waves per workgroup (4 or 8)
  static constexpr int NT = 64 * NW;                // threads per workgroup
  static constexpr int TILE = BS * ROWB;            // bytes of one K (or V) tile
  // LDS ring: two stages (Stage<T, BS, 0/1>); tile u+1 streams in while tile
  // u is used.
  static constexpr int DMA_MAT = BS * CPR / 64 / NW;  // DMA instructions per wave per matrix
  static constexpr int QC = CPR / 2;                // Q chunks per lane
  // key-group merge at the end: round with the most writers has WK/2 of them
  static constexpr int MERGE_O = (WK / 2) * WQ * 16 * 64 * 4;   // 16 O registers per lane
  // row max and row sum: WK/2 writers per query group in the wide rounds,
  // both key groups 0 and 1 in the last one
  static constexpr int MERGE_ML = (WK / 2 > 2 ? WK / 2 : 2) * WQ * 2 * 64 * 4;
  static_assert(DMA_MAT * 64 * NW == BS * CPR, "tile DMA must split evenly over waves");
  static_assert(CPR % 8 == 0, "swizzles act on groups of 8 chunks");
  static_assert(MERGE_O <= TILE, "each half of the merged O must fit in one K or V tile");
};

struct Args {
  const char* q;
  const char* k;
  const char* v;
  const uint8_t* pad;
  const int32_t* rand_idx;
  char* out;
  float* pm;       // [B*H][2][n_s][BS] partial row max (q.k units)
  float* pl;       // [B*H][2][n_s][BS] partial row sum
  float* po;       // [B*H][2][n_s][BS][kD] partial unnormalised output; each 64-row unit
                   // block is stored lane-major (partial_slot())
  float* lse;      // [B*H][L] natural-log row log-sum-exp of the logits, or null (not written)
  int H, L, nb, r, n_s;
  int qmask;       // 1: pairs are masked when the query or the key is padding (pad != null)
  int gc, mc;      // small-problem split (kind 3 units): key chunks per global / middle query
                   // block; 0 when the call runs the ordinary units
};

// LDS ring: one object per (dtype, block, stage) holding that stage's K and V
// tiles.  Distinct objects let the compiler tell a read of one stage from a
// DMA still in flight into another (it tracks only a few DMA targets).
template <typename T, int BS, int S>
struct Stage {
  static __device__ __forceinline__ char* buf() {
    __shared__ __attribute__((aligned(1024))) char b[2 * Cfg<T, BS>::TILE];
    return b;
  }
  static __device__ __forceinline__ char* k() { return buf(); }
  static __device__ __forceinline__ char* v() { return buf() + Cfg<T, BS>::TILE; }
};

// 16-byte chunk swizzles (physical chunk = logical chunk ^ swz(row)).
// K: a score-MFMA operand read hits rows perm_row(0..7) = {R..R+3, R+8..R+11}
//    in one 8-lane phase; this XOR gives them 8 distinct chunk slots.
// V: a transposing read hits 4 consecutive rows x 4 dim quads per 16 lanes;
//    XOR with 2*(row%4) gives the 16 lanes 16 distinct 8-byte slots.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 1; }

// MFMA row i (0..31) -> key / dim offset inside a 32-wide subtile, chosen so
// that accumulator register v of lane group g holds offset
// 16*(v/8) + 8*g + (v%8): two runs of 8 consecutive keys per lane.
__device__ __forceinline__ int perm_row(int i) {
  const int a = i >> 3, gg = (i >> 2) & 1, c = i & 3;
  return 16 * (a >> 1) + 8 * gg + 4 * (a & 1) + c;
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS ring.  The LDS reads of the previous step
// were consumed by MFMAs before this point; DMA writes into a stage are
// ordered by the explicit vmcnt waits.  No memory fence: a fence would drain
// the DMA prefetches that are meant to stay in flight.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier for data exchanged through LDS only: this wave's LDS
// accesses are complete (lgkmcnt = 0), vector-memory operations may stay in
// flight.  (__syncthreads() would also drain them: its fence waits for vmcnt.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0); vmcnt, expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copy key tile `tile` of K and V from HBM straight into LDS stage S.  Each
// DMA instruction moves 64 x 16 bytes; lane l of instruction i fills physical
// chunk slot 64*i + l, so it fetches the logical chunk that the swizzle places
// there.  Rows stay contiguous 128-byte runs.
//
// The DMA instructions are written as asm: the compiler then does not know
// that they write LDS and inserts none of its own (conservative) waits for
// them before LDS accesses.  Every wait for them is explicit: the vmcnt(0) at
// the start of each step, before the workgroup barrier that publishes the tile.
typedef const __attribute__((address_space(1))) char* gchar_ptr;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)p));
}

// Two K and two V DMAs of 64 x 16 bytes each: lane offsets (32-bit) on the
// wave-uniform global bases `kt` / `vt`, into LDS at the wave-uniform
// addresses set in M0 (+16 per lane).  The compiler cannot see that the asm
// reads the bases from a vector-memory instruction, so it inserts no wait
// states for them: an SGPR written by a VALU instruction (v_readlane, e.g.
// reloading a spilled base address) needs 5 before a vector-memory
// instruction reads it.  The leading s_nop 4 gives 5 for every input (none is
// written inside the block); each M0 write gets the 1 it needs.
__device__ __forceinline__ void dma16x4(gchar_ptr kt, gchar_ptr vt, uint32_t ko0, uint32_t vo0, uint32_t ko1,
                                        uint32_t vo1, uint32_t mk0, uint32_t mv0, uint32_t mk1, uint32_t mv1) {
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %8\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %9\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %8\n\t"
      "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %9"
      :
      : "v"(ko0), "v"(vo0), "v"(ko1), "v"(vo1), "s"(mk0), "s"(mv0), "s"(mk1), "s"(mv1), "s"(kt), "s"(vt)
      : "memory", "m0");
}

template <typename T, int BS, int S>
__device__ __forceinline__ void issue_tile(gchar_ptr kbh, gchar_ptr vbh, int tile, int wave, int lane) {
  using C = Cfg<T, BS>;
  const gchar_ptr kt = kbh + static_cast<size_t>(tile) * C::TILE;
  const gchar_ptr vt = vbh + static_cast<size_t>(tile) * C::TILE;
  // (V's address as K's plus the tile size: converting a second generic
  // pointer would cost a null check per DMA group)
  const uint32_t lk = lds_addr(Stage<T, BS, S>::k()), lv = lk + C::TILE;
  static_assert(C::DMA_MAT % 2 == 0, "DMA instructions go in blocks of two per matrix");
  uint32_t ko[C::DMA_MAT], vo[C::DMA_MAT], mk[C::DMA_MAT], mv[C::DMA_MAT];
#pragma unroll
  for (int jj = 0; jj < C::DMA_MAT; ++jj) {
    const int ins = wave + C::NW * jj;
    const int slot = ins * 64 + lane;
    const int row = slot / C::CPR, p = slot % C::CPR;
    ko[jj] = row * C::ROWB + ((p ^ swz_k(row)) << 4);
    vo[jj] = row * C::ROWB + ((p ^ swz_v(row)) << 4);
    mk[jj] = __builtin_amdgcn_readfirstlane(lk + ins * 1024);
    mv[jj] = __builtin_amdgcn_readfirstlane(lv + ins * 1024);
  }
#pragma unroll
  for (int jj = 0; jj < C::DMA_MAT; jj += 2)
    dma16x4(kt, vt, ko[jj], vo[jj], ko[jj + 1], vo[jj + 1], mk[jj], mv[jj], mk[jj + 1], mv[jj + 1]);
}

// Per-wave online-softmax state for 32 query rows (one per lane pair).
struct WaveState {
  f32x16 o[2];   // O^T, dims [0,32) and [32,64)
  float m;       // fp32: running row max in q.k units (may lag the true max by < tau/scale);
                 // bf16: the unit's fixed reference (see softmax_pv)
  float l;       // this lane's part of the row sum
  float qs;      // key offsets apply to this row: 1, or 0 for a padded query row under pair masking
  float big;     // bf16: largest per-subtile probability sum of this lane (the bound check)
};

// V^T operands of one subtile for the PV MFMAs: [dim half][16-key half].
template <typename T>
struct VOp;
template <>
struct VOp<__bf16> {
  bf16x8 a[2][2];
};
template <>
struct VOp<float> {
  float a[2][16];
};

__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 acc, __bf16*) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 acc, float*) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc,
                                               0, 0, 0);
  return acc;
}

typedef const __attribute__((address_space(4))) uint64_t* const_u64_ptr;
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

// S^T = K . Q^T for this wave's 32-key subtile of stage S (no bias yet).
template <typename T, int BS, int S>
__device__ __forceinline__ f32x16 scores(const u32x4 (&qop)[Cfg<T, BS>::QC], int kbase, int lane) {
  using C = Cfg<T, BS>;
  const int j = lane & 31, g = lane >> 5;
  const char* sk = Stage<T, BS, S>::k();
  const int row = kbase + perm_row(j);
  const int sw = swz_k(row);
  u32x4 a[C::QC];
#pragma unroll
  for (int x = 0; x < C::QC; ++x)
    a[x] = *reinterpret_cast<const u32x4*>(sk + row * C::ROWB + (((2 * x + g) ^ sw) << 4));
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int x = 0; x < C::QC; ++x) acc = mfma_qk(a[x], qop[x], acc, static_cast<T*>(nullptr));
  return acc;
}

// The 32 pad bytes of this wave's subtile (wave-uniform, scalar loads).
struct PadWords {
  uint64_t p[4];
};
__device__ __forceinline__ PadWords load_pad(const uint8_t* pad_t, int kbase) {
  const const_u64_ptr pw = (const_u64_ptr)(pad_t + kbase);
  PadWords w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w.p[i] = pw[i];
  return w;
}

// Bit k set iff byte k of w is zero (key padded).  Exact per byte: the high
// bit of (w & 0x7f..) + 0x7f.. never carries across bytes, and the multiply
// gathers the eight flag bits into the top byte (every product term lands on
// a bit of its own, so there are no carries).
__device__ __forceinline__ uint32_t zero_byte_mask(uint64_t w) {
  const uint64_t lo7 = 0x7F7F7F7F7F7F7F7FULL;
  const uint64_t t = ~(((w & lo7) + lo7) | w | lo7);
  return static_cast<uint32_t>(((t >> 7) * 0x0102040810204080ULL) >> 56);
}

// Key bias: -10000 on the logits of padded keys (-80000 in q.k units).  The
// subtile's 32 pad bytes are classified on the scalar unit (wave-uniform):
//   no padded key  -> bias 0, nothing to do (the common case);
//   all 32 padded  -> one uniform bias, returned and folded by the softmax
//                     into its max and exponent offset (no per-key work);
//   mixed          -> the per-key bias enters the score accumulator through
//                     one more product, an fp32 32x32x2 MFMA (one register
//                     per operand): row i of A (key perm_row(i)) carries the
//                     key's bias in k-slot 0 (lanes 0..31), B holds qs there
//                     for every query, k-slot 1 is zero; -80000 * 1 is exact,
//                     so this is the fp32 add of the bias.  Returns 0.
// qs (per lane, i.e. per query row): 1, or 0 for a padded query row under
// pair masking, where every pair of the row gets the offset: a row-uniform
// offset cancels in the softmax, so such a row takes no key offsets at all
// (the caller scales the returned uniform offset by qs too).
// The zero-byte test per word is exact: a byte b sets bit 7 of
// (b - 1) & ~b only when b == 0, and a borrow leaves a byte only from a zero
// byte, which is flagged already.
__device__ __forceinline__ uint64_t zero_bytes_any(uint64_t x) {
  return (x - 0x0101010101010101ull) & ~x & 0x8080808080808080ull;
}

// No key of the subtile padded (no pad byte zero).  Tested first on the AND of
// the four words: a byte of the AND is non-zero only if that byte is non-zero
// in every word, so a zero-free AND settles the common all-valid case in half
// the scalar instructions; otherwise (a zero byte somewhere, or non-0/1 bytes
// whose AND vanishes) the exact per-word test decides.
__device__ __forceinline__ bool no_key_padded(const PadWords& w) {
  if (zero_bytes_any(w.p[0] & w.p[1] & w.p[2] & w.p[3]) == 0) return true;
  return (zero_bytes_any(w.p[0]) | zero_bytes_any(w.p[1]) | zero_bytes_any(w.p[2]) | zero_bytes_any(w.p[3])) == 0;
}

__device__ __forceinline__ float apply_pad(f32x16& acc, const PadWords& w, int lane, float qs = 1.0f) {
  if (no_key_padded(w)) return 0.0f;
  if ((w.p[0] | w.p[1] | w.p[2] | w.p[3]) == 0) return kMaskRaw;
  const uint32_t m = zero_byte_mask(w.p[0]) | (zero_byte_mask(w.p[1]) << 8) |
                     (zero_byte_mask(w.p[2]) << 16) | (zero_byte_mask(w.p[3]) << 24);
  const int j = lane & 31;
  const bool lo = lane < 32;                        // lanes holding k-slot 0
  const bool padded = (m >> perm_row(j)) & 1u;
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(lo && padded ? kMaskRaw : 0.0f, lo ? qs : 0.0f, acc, 0, 0, 0);
  return 0.0f;
}

// V^T operands of this wave's subtile of stage S.
template <typename T, int BS, int S>
__device__ __forceinline__ VOp<T> load_v(int kbase, int lane) {
  using C = Cfg<T, BS>;
  const char* sv = Stage<T, BS, S>::v();
  VOp<T> vo;
  if constexpr (sizeof(T) == 2) {
    // Transposing LDS reads (ds_read_b64_tr_b16): lane (dim, g) gets V[key][dim]
    // for 4 consecutive keys; lanes 4e+m of each 16-lane group address row
    // key0+e at dim quad m.  Rows key0 + {0, 4, 16, 20} share the swizzle
    // (it depends on row % 4).
    const int g = lane >> 5, e4 = (lane >> 2) & 3;
    const int r0 = kbase + 8 * g + e4;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const int dstart = dh * 32 + perm_row(16 * ((lane >> 4) & 1) + 4 * (lane & 3));
      const int dchunk = dstart >> 3, dbyte = (dstart & 7) * 2;
      const char* base = sv + r0 * C::ROWB + ((dchunk ^ swz_v(r0)) << 4) + dbyte;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + 16 * mm * C::ROWB));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + (16 * mm + 4) * C::ROWB));
        vo.a[dh][mm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  } else {
    const int j = lane & 31, g = lane >> 5;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const int dim = dh * 32 + perm_row(j);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kbase + 16 * (v >> 3) + 8 * g + (v & 7);
        vo.a[dh][v] = *reinterpret_cast<const float*>(
            sv + key * C::ROWB + (((dim >> 2) ^ swz_v(key)) << 4) + (dim & 3) * 4);
      }
    }
  }
  return vo;
}

// Max of this lane's 16 scores of the subtile and `m0`.
__device__ __forceinline__ float lane_max(const f32x16& acc, float m0) {
  float m8[6];
  m8[0] = fmaxf(fmaxf(acc[0], acc[1]), acc[2]);
  m8[1] = fmaxf(fmaxf(acc[3], acc[4]), acc[5]);
  m8[2] = fmaxf(fmaxf(acc[6], acc[7]), acc[8]);
  m8[3] = fmaxf(fmaxf(acc[9], acc[10]), acc[11]);
  m8[4] = fmaxf(fmaxf(acc[12], acc[13]), acc[14]);
  m8[5] = fmaxf(acc[15], m0);
  return fmaxf(fmaxf(fmaxf(m8[0], m8[1]), m8[2]), fmaxf(fmaxf(m8[3], m8[4]), m8[5]));
}

// Row max of this subtile's 16 scores per lane (and `m0`), over both lane
// halves (the two 16-key halves of the query row).
__device__ __forceinline__ float subtile_max(const f32x16& acc, float m0) {
  const float m = lane_max(acc, m0);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

constexpr int kTile64 = 64 * kD * 2;               // one 64-key bf16 tile of K (or V): 8 KiB
constexpr float kProbBound = 4294967296.0f;        // 2^32: the largest probability the fast path keeps

// Probabilities of one 32-key subtile against the reference m (q.k units)
// and uniform offset `bias`: P = 2^((s + bias - m) c), rounded to the bf16
// PV operands; returns this lane's sum of the rounded values.
__device__ __forceinline__ float probs_w(const f32x16& s, float m, float bias, bf16x8 (&pb)[2]) {
  const float mc = (m - bias) * kScaleLog2;
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float lsum = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      f32x2 pr = {__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h + e], kScaleLog2, -mc)),
                  __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h + e + 1], kScaleLog2, -mc))};
      const bf16x2 c2 = __builtin_convertvector(pr, bf16x2);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(c2, ones, lsum, false);
      pb[h][e] = c2[0];
      pb[h][e + 1] = c2[1];
    }
  return lsum;
}

// O^T += V^T P^T for one subtile (4 MFMAs: 2 dim halves x 2 16-key halves).
template <typename WS>
__device__ __forceinline__ void pv_w(WS& ws, const VOp<__bf16>& vo, const bf16x8 (&pb)[2]) {
#pragma unroll
  for (int mm = 0; mm < 2; ++mm)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
      ws.o[dh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vo.a[dh][mm], pb[mm], ws.o[dh], 0, 0, 0);
}

// Online softmax of one score subtile (lane = query row, 16 of its 32 keys)
// and O^T += V^T . P^T.  Registers only.  `first`: the unit's first tile
// (wave-uniform), whose max starts the running max.  `bias` (wave-uniform, 0
// or the padding bias): added to every score of the subtile, through the max
// and the exponent offset rather than per score.
template <typename T>
__device__ __forceinline__ void softmax_pv(WaveState& ws, const f32x16& acc, const VOp<T>& vo, bool first,
                                           float bias) {
  if constexpr (sizeof(T) == 2) {
    // bf16: every probability of the unit is taken against one fixed
    // reference, the row max of this wave's keys of the unit's first tile
    // (the reading of the block-128 kernel: P <= 2^32 is checked per subtile
    // through the lane's probability sum, and a unit that exceeds it is
    // recomputed exactly at its end); no max and no rescale in the step.
    if (first) ws.m = subtile_max(acc, acc[15]) + bias;
    bf16x8 pb[2];
    const float lsum = probs_w(acc, ws.m, bias, pb);
    ws.l += lsum;
    ws.big = fmaxf(ws.big, lsum);
    pv_w(ws, vo, pb);
  } else {
    // P = 2^((s + bias - m) c) against the running max m first; the tile's own
    // max is reduced meanwhile, and only if it exceeds m by more than tau/c
    // (rare) are O and l rescaled and P recomputed.  Keeps the exps off the
    // critical path of the max reduction.
    if (first) ws.m = subtile_max(acc, acc[15]) + bias;
    float p[16];
    float mc = (ws.m - bias) * kScaleLog2;
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kScaleLog2, -mc));
    // Each lane tests its own 16 scores; only a rescale needs the row max over
    // both lane halves.
    const float lm = lane_max(acc, acc[15]) + bias;
    if (__any(lm - ws.m > kRescaleTau / kScaleLog2)) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lm), __float_as_uint(lm), false, false);
      const float mloc = fmaxf(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])), ws.m);
      const float alpha = __builtin_amdgcn_exp2f((ws.m - mloc) * kScaleLog2);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        ws.o[0][v] *= alpha;
        ws.o[1][v] *= alpha;
      }
      ws.l *= alpha;
      ws.m = mloc;
      mc = (ws.m - bias) * kScaleLog2;
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kScaleLog2, -mc));
    }
    float lsum = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) lsum += p[v];
    ws.l += lsum;
#pragma unroll
    for (int v = 0; v < 16; ++v)
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
        ws.o[dh] = __builtin_amdgcn_mfma_f32_32x32x2f32(vo.a[dh][v], p[v], ws.o[dh], 0, 0, 0);
  }
}

// Key tiles of a work unit, computed on the fly (all values wave-uniform).
// (No bool members and no padding: these structs are copied around the unit
// loop, and padding bytes would leave a small private object behind.)
struct TileList {
  int first;             // global unit: first tile of its chunk; middle unit: band start
  int nwin;              // middle unit: band blocks inside 1..nb-2
  int nb;
  int global;            // 1: global unit, 0: middle unit
  int skip;              // middle unit: position of its first tile in the block's list
                         // (non-zero only for the key chunks of kind 3 units)
  int r;                 // middle unit: random blocks per row (entries of `rand`); 0 otherwise
  const_i32_ptr rand;    // middle unit: its row of the random-block table
};

__device__ __forceinline__ int tile_at(const TileList& tl, int u) {
  if (tl.global) return tl.first + u;
  u += tl.skip;
  if (u == 0) return 0;
  if (u <= tl.nwin) return tl.first + u - 1;
  if (u == tl.nwin + 1) return tl.nb - 1;
  int e = tl.rand[u - tl.nwin - 2];
  return e < 1 ? 1 : (e > tl.nb - 2 ? tl.nb - 2 : e);   // never read outside the sequence
}

// This lane's id, computed where the call stands (volatile asm: not hoisted
// out of a loop, so no register holds it across one).
__device__ __forceinline__ int lane_id_here() {
  int x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

// tile_at() for 64 list positions at once, one per lane: lane j gets the tile
// of position u + j (positions at or past the list's end get some tile inside
// the sequence; the caller never uses them).  Selects instead of branches, and
// one vector load of the random-table row, bounded by the row's length,
// instead of one dependent scalar load per random position; the steps then
// take their ids with one lane read each.
__device__ __forceinline__ int tile_ids(const TileList& tl, int u, int lane) {
  const int p = u + lane;
  if (tl.global) return tl.first + p;
  const int q = p + tl.skip;
  int t = q == 0 ? 0 : (q <= tl.nwin ? tl.first + q - 1 : tl.nb - 1);
  if (tl.r > 0) {
    // a buffer load bounded by the row (4 r bytes): an entry index outside
    // [0, r) (positions before or after the random part) reads 0 instead of
    // memory.  Descriptor word 3: 32-bit data format, no swizzle, no stride.
    const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
        (void*)reinterpret_cast<uintptr_t>(tl.rand), 0, 4 * tl.r, 0x00020000);
    int e = __builtin_amdgcn_raw_buffer_load_b32(row, 4 * (q - tl.nwin - 2), 0, 0);
    e = e < 1 ? 1 : (e > tl.nb - 2 ? tl.nb - 2 : e);   // never read outside the sequence
    t = q > tl.nwin + 1 ? e : t;
  }
  return t;
}

// A decoded work unit (all values wave-uniform).  Per (b, h) the units are the
// global units (block 0 chunks, then block nb-1 chunks; QSPLIT row slices
// each) followed by the middle units (nb-2 blocks, QSPLIT row slices each).
// `kind` selects which of them a grid covers: 0 = all, 1 = global units only,
// 2 = middle units only.  A unit covers query rows [q0, q0 + 64) of (b, h).
// gsel < 0: a middle query block, finalised in place.  gsel in {0, 1}: global
// query block 0 or nb-1 against one key chunk of the split-K, written as a
// partial for the merge kernel.
// kind 3 (problems with too few units to fill the chip): every query block is
// split over its key tiles -- a->gc chunks per global block, a->mc per middle
// block, each a contiguous run of the block's tile list -- and every unit
// writes a partial (gsel 2 for the middle ones); the merge kernel then
// combines the chunks of every query block.  Partial slots per (b, h):
// [block 0 chunks | block nb-1 chunks | middle block 1 chunks | ...].
struct Unit {
  size_t off;            // byte offset of (b, h) in q, k, v and out: bh * L * ROWB
  size_t pbase;          // global unit: partial row index of its first query row
  int b, q0, gsel, ntiles;
  TileList tl;
};

// Kernel arguments read straight from the kernel-argument segment where they
// are used.  The empty asm makes the pointer opaque, so the loads are not
// hoisted and the arguments do not occupy scalar registers across the tile
// loop (they are needed only at unit boundaries).
typedef const __attribute__((address_space(4))) Args* kargs_ptr;
__device__ __forceinline__ kargs_ptr kargs() {
  kargs_ptr p = (kargs_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

template <typename T, int BS, int kind>
__device__ __forceinline__ int units_per_bh(kargs_ptr a) {
  constexpr int QS = Cfg<T, BS>::QSPLIT;
  if constexpr (kind == 3) return (2 * a->gc + (a->nb - 2) * a->mc) * QS;
  return (kind == 2 ? 0 : 2 * a->n_s * QS) + (kind == 1 ? 0 : (a->nb - 2) * QS);
}

// Position of a unit, kept incrementally so that the unit loop does no
// integer division: unit = bh * per_bh + u, bh = b * H + h.
struct Cursor {
  int unit, bh, u, b, h;
};

template <typename T, int BS, int kind>
__device__ __forceinline__ Cursor cursor_at(kargs_ptr a, int unit) {
  const int per_bh = units_per_bh<T, BS, kind>(a);
  Cursor c;
  c.unit = unit;
  c.bh = unit / per_bh;
  c.u = unit - c.bh * per_bh;
  c.b = c.bh / a->H;
  c.h = c.bh - c.b * a->H;
  return c;
}

template <typename T, int BS, int kind>
__device__ __forceinline__ Cursor cursor_advance(kargs_ptr a, Cursor c, int stride) {
  const int per_bh = units_per_bh<T, BS, kind>(a), H = a->H;
  c.unit += stride;
  c.u += stride;
  while (c.u >= per_bh) {
    c.u -= per_bh;
    ++c.bh;
    if (++c.h == H) {
      c.h = 0;
      ++c.b;
    }
  }
  return c;
}

template <typename T, int BS, int kind>
__device__ __forceinline__ Unit decode_unit(kargs_ptr a, const Cursor& c) {
  using C = Cfg<T, BS>;
  constexpr int QS = C::QSPLIT;
  constexpr int LQS = QS == 2 ? 1 : 0;
  static_assert(QS == 1 || QS == 2, "row slices per query block");
  const int nb = a->nb, n_s = a->n_s;
  Unit w;
  w.off = static_cast<size_t>(c.bh) * a->L * C::ROWB;
  w.b = c.b;
  w.tl.nb = nb;
  w.tl.skip = 0;
  if constexpr (kind == 3) {
    const int gc = a->gc, mc = a->mc;
    const size_t slots = static_cast<size_t>(2 * gc + (nb - 2) * mc);   // partial blocks per (b, h)
    int slot, qb, qh;
    if (c.u < 2 * gc * QS) {
      const int half = gc * QS;
      w.gsel = c.u >= half ? 1 : 0;
      const int rem = c.u - (w.gsel ? half : 0);
      const int chunk = rem >> LQS;
      qh = rem & (QS - 1);
      qb = w.gsel ? nb - 1 : 0;
      slot = w.gsel * gc + chunk;
      w.tl.global = 1;
      w.tl.first = chunk * nb / gc;                // balanced chunks: none is empty (gc <= nb)
      w.ntiles = (chunk + 1) * nb / gc - w.tl.first;
      w.tl.nwin = 0;
      w.tl.r = 0;
      w.tl.rand = nullptr;
    } else {
      const int v = (c.u - 2 * gc * QS) >> LQS;
      qh = (c.u - 2 * gc * QS) & (QS - 1);
      const int mi = v / mc, chunk = v - mi * mc;
      qb = mi + 1;
      w.gsel = 2;
      slot = 2 * gc + mi * mc + chunk;
      const int lo = qb - 1 < 1 ? 1 : qb - 1;
      const int hi = qb + 1 > nb - 2 ? nb - 2 : qb + 1;
      const int r = a->r;
      w.tl.global = 0;
      w.tl.first = lo;
      w.tl.nwin = hi - lo + 1;
      w.tl.r = r;
      w.tl.rand = (const_i32_ptr)(a->rand_idx + (static_cast<size_t>(c.h) * (nb - 2) + (qb - 1)) * r);
      const int nt = 2 + w.tl.nwin + r;            // mc <= the fewest tiles of any middle block
      w.tl.skip = chunk * nt / mc;
      w.ntiles = (chunk + 1) * nt / mc - w.tl.skip;
    }
    w.q0 = qb * BS + qh * C::QROWS;
    w.pbase = (static_cast<size_t>(c.bh) * slots + slot) * BS + qh * C::QROWS;
    return w;
  }
  const int n_g = kind == 2 ? 0 : 2 * n_s * QS;
  if (c.u < n_g) {
    const int half = n_s * QS;
    w.gsel = c.u >= half ? 1 : 0;
    const int rem = c.u - (w.gsel ? half : 0);
    const int chunk = rem >> LQS, qh = rem & (QS - 1);
    w.q0 = (w.gsel ? nb - 1 : 0) * BS + qh * C::QROWS;
    w.pbase = ((static_cast<size_t>(c.bh) * 2 + w.gsel) * n_s + chunk) * BS + qh * C::QROWS;
    w.tl.global = 1;
    w.tl.first = chunk * kChunkTiles;
    w.tl.nwin = 0;
    w.tl.r = 0;
    w.tl.rand = nullptr;
    w.ntiles = nb - w.tl.first < kChunkTiles ? nb - w.tl.first : kChunkTiles;
  } else {
    w.gsel = -1;
    const int v = c.u - n_g;
    const int qb = (v >> LQS) + 1, qh = v & (QS - 1);
    w.q0 = qb * BS + qh * C::QROWS;
    w.pbase = 0;
    const int lo = qb - 1 < 1 ? 1 : qb - 1;          // band without the global blocks
    const int hi = qb + 1 > nb - 2 ? nb - 2 : qb + 1;
    w.tl.global = 0;
    w.tl.first = lo;
    w.tl.nwin = hi - lo + 1;
    const int r = a->r;
    w.tl.r = r;
    w.tl.rand = (const_i32_ptr)(a->rand_idx + (static_cast<size_t>(c.h) * (nb - 2) + (qb - 1)) * r);
    w.ntiles = 2 + w.tl.nwin + r;
  }
  return w;
}

// This wave's 32 query rows as the B operand of the score products; `qrow`
// points at the unit's first query row.
template <typename T, int BS>
__device__ __forceinline__ void load_q(const char* qrow0, int wq, int lane, u32x4 (&qop)[Cfg<T, BS>::QC]) {
  using C = Cfg<T, BS>;
  const char* qrow = qrow0 + static_cast<size_t>(wq * 32 + (lane & 31)) * C::ROWB;
#pragma unroll
  for (int x = 0; x < C::QC; ++x)
    qop[x] = *reinterpret_cast<const u32x4*>(qrow + (2 * x + (lane >> 5)) * 16);
}

// What the last step of a unit needs to prefetch the next unit (its K, V and
// Q addresses are rebuilt from the kernel arguments there, once per unit).
struct NextUnit {
  size_t off;            // its (b, h) byte offset
  int q0;                // its first query row
  int tile0;             // its first key tile
  int pf;                // 1: prefetch (the current unit has an even tile count and a successor)
  int unused;
};

// Step u of the tile loop: tile u sits in stage S = u % 2; tile_u and
// tile_fill are the ids of tiles u and u+1.  On the last step of a unit with
// an even tile count (S == 1) the next unit is prefetched: its tile 0 into
// stage 0 and, once this step's score products have consumed Q, its Q rows
// into qop.
template <typename T, int BS, int S, bool HAS_PAD>
__device__ __forceinline__ void step(WaveState& ws, u32x4 (&qop)[Cfg<T, BS>::QC], bool first, bool last,
                                     int tile_u, int tile_fill, gchar_ptr kbh, gchar_ptr vbh,
                                     const uint8_t* pad_b, int wave, int lane, int kbase,
                                     const NextUnit& nx, int wq) {
  // This wave's DMA of tile u has landed and its LDS reads of the previous
  // step are complete (vmcnt = lgkmcnt = 0; on a unit's first step this also
  // covers the previous unit's output stores); after the barrier every wave's
  // part of tile u is visible and the stage of tile u-1 is free to refill.
  // The pad bytes of tile u are loaded first, so that their scalar load
  // completes under this wait and the barrier: scalar and LDS loads share one
  // counter and scalar loads may return out of order, so an outstanding one
  // would turn every later LDS wait of the step into a full drain.
  PadWords pw;
  if constexpr (HAS_PAD) {
    pw = load_pad(pad_b + static_cast<size_t>(tile_u) * BS, kbase);
    asm volatile("" ::: "memory");
  }
  __builtin_amdgcn_s_waitcnt(7 << 4);
  ring_barrier();
  // Critical path first: K reads and the score products.  The V^T reads and
  // the DMA of the next tile are issued while the products run.
  f32x16 s = scores<T, BS, S>(qop, kbase, lane);
  const VOp<T> vo = load_v<T, BS, S>(kbase, lane);
  if (!last) {
    issue_tile<T, BS, S ^ 1>(kbh, vbh, tile_fill, wave, lane);
  } else if (S == 1 && nx.pf) {
    const kargs_ptr a = kargs();
    issue_tile<T, BS, 0>((gchar_ptr)(a->k) + nx.off, (gchar_ptr)(a->v) + nx.off, nx.tile0, wave, lane);
  }
  float pbias = 0.0f;
  if constexpr (HAS_PAD) pbias = apply_pad(s, pw, lane, ws.qs) * ws.qs;
  if (S == 1 && last && nx.pf) {
    // Q is dead after the score products: refill it for the next unit.  The
    // empty asm ties the loads after those products.
    asm volatile("" : "+v"(s) : : "memory");
    load_q<T, BS>(kargs()->q + nx.off + static_cast<size_t>(nx.q0) * Cfg<T, BS>::ROWB, wq, lane, qop);
  }
  softmax_pv<T>(ws, s, vo, first, pbias);
}

__device__ __forceinline__ void store_row8(char* dst, const float* x, __bf16*) {
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    f32x2 pr = {x[e], x[e + 1]};
    bf16x2 c2 = __builtin_convertvector(pr, bf16x2);
    o[e] = c2[0];
    o[e + 1] = c2[1];
  }
  *reinterpret_cast<bf16x8*>(dst) = o;
}
__device__ __forceinline__ void store_row8(char* dst, const float* x, float*) {
  f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
  reinterpret_cast<f32x4*>(dst)[0] = lo;
  reinterpret_cast<f32x4*>(dst)[1] = hi;
}

__device__ __forceinline__ void store_f32x4(char* dst, f32x4 x, __bf16*) {
  f32x2 a = {x[0], x[1]}, b = {x[2], x[3]};
  bf16x2 ca = __builtin_convertvector(a, bf16x2), cb = __builtin_convertvector(b, bf16x2);
  __bf16 o[4] = {ca[0], ca[1], cb[0], cb[1]};
  *reinterpret_cast<uint64_t*>(dst) = __builtin_bit_cast(uint64_t, o);
}
__device__ __forceinline__ void store_f32x4(char* dst, f32x4 x, float*) {
  *reinterpret_cast<f32x4*>(dst) = x;
}

// Row max / row sum exchange area of the key-group merge.
template <typename T, int BS>
struct MergeML {
  static __device__ __forceinline__ float* buf() {
    __shared__ float b[Cfg<T, BS>::MERGE_ML / 4];
    return b;
  }
};

// Float offset, inside a 64-row x 64-dim partial block of a global unit, of
// the 4 dims [32 keep + 16 (q / 2) + 8 g + 4 (q % 2), +4) of row 32 wq + j,
// where lane = j + 32 g: blocks of 64 lanes x 4 floats per (wq, keep, q), so
// that a wave's store of one q is 1 KB contiguous.
__device__ __forceinline__ int partial_slot(int wq, int keep, int q, int lane) {
  return ((wq * 2 + keep) * 4 + q) * 256 + lane * 4;
}

// Last merge round for key group KEEP (0 or 1) of one query group: see
// finalize().
template <typename T, int BS, int KEEP>
__device__ __forceinline__ void finalize_half(WaveState& ws, const Unit& w, int wq, int lane, float* mo0, float* mo1,
                                              float* mml) {
  using C = Cfg<T, BS>;
  constexpr int GIVE = KEEP ^ 1;
  {
    float* mo_give = GIVE ? mo1 : mo0;
#pragma unroll
    for (int v = 0; v < 16; ++v) mo_give[(wq * 16 + v) * 64 + lane] = ws.o[GIVE][v];
    mml[((wq * 2 + KEEP) * 2) * 64 + lane] = ws.m;
    mml[((wq * 2 + KEEP) * 2 + 1) * 64 + lane] = ws.l;
  }
  lds_barrier();
  const int j = lane & 31, g = lane >> 5;
  const float m1 = mml[((wq * 2 + GIVE) * 2) * 64 + lane], l1 = mml[((wq * 2 + GIVE) * 2 + 1) * 64 + lane];
  const float mm = fmaxf(ws.m, m1);
  float a0 = __builtin_amdgcn_exp2f((ws.m - mm) * kScaleLog2);
  float a1 = __builtin_amdgcn_exp2f((m1 - mm) * kScaleLog2);
  const float lh = ws.l * a0 + l1 * a1;             // this lane half's share of the row sum
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lh), __float_as_uint(lh), false, false);
  const float l = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);   // both lane halves of the row
  char* dst;
  float* pm = nullptr;
  float* pl = nullptr;
  size_t pidx = 0;
  if (w.gsel < 0) {
    const float inv = __builtin_amdgcn_rcpf(l);   // 1 ulp
    a0 *= inv;
    a1 *= inv;
    dst = kargs()->out + w.off + static_cast<size_t>(w.q0 + wq * 32 + j) * C::ROWB;
    float* lse = kargs()->lse;
    if (KEEP == 0 && g == 0 && lse != nullptr)   // LSE = m / sqrt(d) + ln(l)
      lse[w.off / C::ROWB + w.q0 + wq * 32 + j] = (mm * kScaleLog2 + __builtin_amdgcn_logf(l)) * kLn2;
  } else {
    const kargs_ptr a = kargs();
    pidx = w.pbase + wq * 32 + j;
    dst = reinterpret_cast<char*>(a->po + pidx * kD);
    pm = a->pm;
    pl = a->pl;
  }
  const float* mo_keep = KEEP ? mo1 : mo0;
  float x[2][8];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      x[h8][e] = ws.o[KEEP][8 * h8 + e] * a0 + mo_keep[(wq * 16 + 8 * h8 + e) * 64 + lane] * a1;
  if (w.gsel < 0) {
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
      store_row8(dst + (KEEP * 32 + 16 * h8 + 8 * g) * C::ES, x[h8], static_cast<T*>(nullptr));
    return;
  }
  // Partial O, lane-major inside the unit's 64 x 64 block: every store writes
  // 1 KB contiguous (layout in partial_slot()).
  float* blk = reinterpret_cast<float*>(dst) - static_cast<size_t>(wq * 32 + j) * kD;
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 v4 = {x[h8][4 * hf], x[h8][4 * hf + 1], x[h8][4 * hf + 2], x[h8][4 * hf + 3]};
      *reinterpret_cast<f32x4*>(blk + partial_slot(wq, KEEP, 2 * h8 + hf, lane)) = v4;
    }
  if (KEEP == 0 && g == 0) {
    pm[pidx] = mm;
    pl[pidx] = l;
  }
}

// End of a unit: merge the key groups of each query group (tree over LDS,
// O through stage S -- the stage of the unit's last tile -- and (max, sum)
// through MergeML), then write the output rows (middle unit) or the partial
// (global unit).  Key groups 0 and 1 finish the last round together, each
// on half of the head dims; for a middle unit the division by the row sum is
// folded into the two merge weights.
template <typename T, int BS, int S>
__device__ __forceinline__ void finalize(WaveState& ws, const Unit& w, int wq, int wk, int lane) {
  using C = Cfg<T, BS>;
  float* mo0 = reinterpret_cast<float*>(Stage<T, BS, S>::k());
  float* mo1 = reinterpret_cast<float*>(Stage<T, BS, S>::v());
  float* mml = MergeML<T, BS>::buf();
  // rounds with more than one receiving key group (4 key groups: 2,3 -> 0,1)
#pragma unroll
  for (int stride = C::WK / 2; stride >= 2; stride /= 2) {
    lds_barrier();
    if (wk >= stride && wk < 2 * stride) {
      const int slot = (wk - stride) * C::WQ + wq;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        mo0[(slot * 16 + v) * 64 + lane] = ws.o[0][v];
        mo1[(slot * 16 + v) * 64 + lane] = ws.o[1][v];
      }
      mml[(slot * 2) * 64 + lane] = ws.m;
      mml[(slot * 2 + 1) * 64 + lane] = ws.l;
    }
    lds_barrier();
    if (wk < stride) {
      const int slot = wk * C::WQ + wq;
      const float m1 = mml[(slot * 2) * 64 + lane], l1 = mml[(slot * 2 + 1) * 64 + lane];
      const float mm = fmaxf(ws.m, m1);
      const float a0 = __builtin_amdgcn_exp2f((ws.m - mm) * kScaleLog2);
      const float a1 = __builtin_amdgcn_exp2f((m1 - mm) * kScaleLog2);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        ws.o[0][v] = ws.o[0][v] * a0 + mo0[(slot * 16 + v) * 64 + lane] * a1;
        ws.o[1][v] = ws.o[1][v] * a0 + mo1[(slot * 16 + v) * 64 + lane] * a1;
      }
      ws.l = ws.l * a0 + l1 * a1;
      ws.m = mm;
    }
  }
  // Last round, between key groups 0 and 1, split by head dims: wave wk
  // keeps dims [32 wk, 32 wk + 32) (its o[wk]) and hands the other half to
  // its partner through stage S (o[0] halves in the K part, o[1] halves in
  // the V part); both publish (max, sum).  Each then merges and writes its
  // half, so the two waves finish together.  (Wave-uniform branch on wk, so
  // the register arrays are indexed by constants only.)
  lds_barrier();
  if (wk == 0)
    finalize_half<T, BS, 0>(ws, w, wq, lane, mo0, mo1, mml);
  else if (wk == 1)
    finalize_half<T, BS, 1>(ws, w, wq, lane, mo0, mo1, mml);
  else
    lds_barrier();   // key groups 2 and 3 (block 128) are merged already: the round's second barrier
}


// A wave's softmax state per query row (fixed-reference softmax).
struct WaveStateW {
  f32x16 o[2];     // O^T, dims [0,32) and [32,64)
  float m;         // the unit's reference max (q.k units)
  float l;         // this lane's part of the row sum
  float big;       // largest per-subtile probability sum of this lane (the bound check)
  float qs;        // key offsets apply to this row: 1, or 0 for a padded query row under pair masking
};

// Pad offsets of one 32-key subtile, classified on the scalar unit before the
// score products (the classes of apply_pad()): the uniform offset `bias` (0,
// or -10000 on the logit when all 32 keys are padding) and, for a subtile
// with both kinds of keys, `mixed` = the per-key mask (bit k: key k padded),
// added after the products by add_pad_bias(); 0 otherwise.
struct PadClass {
  float bias;
  uint32_t mixed;
};
__device__ __forceinline__ PadClass classify_pad(const PadWords& w) {
  PadClass c;
  c.bias = 0.0f;
  c.mixed = 0u;
  if (no_key_padded(w)) return c;
  if ((w.p[0] | w.p[1] | w.p[2] | w.p[3]) == 0) {
    c.bias = kMaskRaw;
    return c;
  }
  c.mixed = zero_byte_mask(w.p[0]) | (zero_byte_mask(w.p[1]) << 8) | (zero_byte_mask(w.p[2]) << 16) |
            (zero_byte_mask(w.p[3]) << 24);
  return c;
}

// The per-key offsets of a mixed subtile, added to the score accumulator by
// one fp32 32x32x2 MFMA (as in apply_pad(), with its per-query factor qs).
__device__ __forceinline__ void add_pad_bias(f32x16& acc, uint32_t mixed, int lane, float qs) {
  const int j = lane & 31;
  const bool lo = lane < 32;
  const bool padded = (mixed >> perm_row(j)) & 1u;
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(lo && padded ? kMaskRaw : 0.0f, lo ? qs : 0.0f, acc, 0, 0, 0);
}

// 64-key tile id of entry i of a unit's tile list (block-level list, TPB
// 64-key tiles per key block).
template <int TPB>
__device__ __forceinline__ int tile64_at(const TileList& tl, int i) {
  if constexpr (TPB == 1) return tile_at(tl, i);
  return TPB * tile_at(tl, i / TPB) + i % TPB;
}

// Scores of one 32-key subtile read straight from global memory (the slow
// path): S^T = K Q^T with K rows perm_row-ordered as in scores(), the
// subtile's pad offsets added per key in fp32 (times the row's factor qs).
__device__ __forceinline__ f32x16 scores_global(const char* kt, const uint8_t* pt, const u32x4 (&qop)[4], int kbase,
                                                int lane, float qs) {
  const int j = lane & 31, g = lane >> 5;
  const char* krow = kt + (kbase + perm_row(j)) * (kD * 2);
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x)
    acc = mfma_qk(*reinterpret_cast<const u32x4*>(krow + (2 * x + g) * 16), qop[x], acc, static_cast<__bf16*>(nullptr));
  if (pt != nullptr) {
#pragma unroll
    for (int v = 0; v < 16; ++v)   // element v holds key kbase + 16 (v / 8) + 8 g + v % 8
      if (pt[kbase + 16 * (v >> 3) + 8 * g + (v & 7)] == 0) acc[v] += kMaskRaw * qs;
  }
  return acc;
}

// Slow path of a unit in which some lane of this wave saw a probability sum
// above the bound: this wave's state over its keys of the unit is recomputed
// exactly, in two passes over the unit's tiles read straight from global
// memory -- the row max over every allowed key first, then the
// probabilities against it (all at most 1) and O, l.  Registers and global
// loads only (no LDS, no barrier), so the other waves of the workgroup do not
// take part.  The wave's keys: NKB 32-key halves of every 64-key tile from
// key kb0 (NKB 2: complete rows; NKB 1: the key group of kb0).
template <int TPB, bool HAS_PAD, int NKB, typename WS>
__device__ __forceinline__ void redo_unit_w(WS& ws, const Unit& cu, int ntiles, int wq, int lane, int kb0) {
  const kargs_ptr a = kargs();
  const char* kbh = a->k + cu.off;
  const char* vbh = a->v + cu.off;
  const uint8_t* pad_b = HAS_PAD ? a->pad + static_cast<size_t>(cu.b) * a->L : nullptr;
  u32x4 q[4];
  load_q<__bf16, 64>(a->q + cu.off + static_cast<size_t>(cu.q0) * (kD * 2), wq, lane, q);
  float lm = -__builtin_inff();
#pragma unroll 1
  for (int i = 0; i < NKB * ntiles; ++i) {
    const int t = tile64_at<TPB>(cu.tl, i / NKB), kb = kb0 + 32 * (i % NKB);
    const char* kt = kbh + static_cast<size_t>(t) * kTile64;
    const uint8_t* pt = HAS_PAD ? pad_b + static_cast<size_t>(t) * 64 : nullptr;
    lm = lane_max(scores_global(kt, pt, q, kb, lane, ws.qs), lm);
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lm), __float_as_uint(lm), false, false);
  ws.m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  ws.l = 0.0f;
  ws.big = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    ws.o[0][v] = 0.0f;
    ws.o[1][v] = 0.0f;
  }
  const int j = lane & 31, g = lane >> 5;
#pragma unroll 1
  for (int i = 0; i < NKB * ntiles; ++i) {
    const int t = tile64_at<TPB>(cu.tl, i / NKB), kb = kb0 + 32 * (i % NKB);
    const char* kt = kbh + static_cast<size_t>(t) * kTile64;
    const uint8_t* pt = HAS_PAD ? pad_b + static_cast<size_t>(t) * 64 : nullptr;
    const f32x16 s = scores_global(kt, pt, q, kb, lane, ws.qs);
    bf16x8 pb[2];
    ws.l += probs_w(s, ws.m, 0.0f, pb);
    // V^T operand: dim dh*32 + perm_row(j), keys kb + 16 mm + 8 g + e (e = 0..7),
    // gathered two keys at a time
    const uint16_t* vcol = reinterpret_cast<const uint16_t*>(vbh + static_cast<size_t>(t) * kTile64) +
                           (kb + 8 * g) * kD + perm_row(j);
    VOp<__bf16> vo;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const uint16_t* c = vcol + 16 * mm * kD + 32 * dh;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = static_cast<uint32_t>(c[(2 * e) * kD]) | (static_cast<uint32_t>(c[(2 * e + 1) * kD]) << 16);
        vo.a[dh][mm] = __builtin_bit_cast(bf16x8, w);
      }
    pv_w(ws, vo, pb);
  }
}

// A persistent workgroup: it runs a fixed sequence of work units back to back,
// streaming their key tiles through the 2-stage LDS ring.  The sequence: the
// hardware deals workgroup ids round robin to the 8 XCDs, so workgroup x runs
// on XCD x % 8; each XCD owns a contiguous range of units (one (batch, head)
// after another, which keeps their K/V in that XCD's L2) and its workgroups
// take every (G/8)-th unit of it.  While the last tile of a unit is processed
// the next unit's first tile and Q rows are already being fetched, so a unit
// start waits for nothing but the stores of the previous one.
template <typename T, int BS, int kind, bool HAS_PAD>
__device__ __forceinline__ void run(int n_units) {
  using C = Cfg<T, BS>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave % C::WQ, wk = wave / C::WQ;
  const int kbase = wk * 32;             // this wave's 32 keys of every tile

  int first, stride, end;
  {
    const int G = gridDim.x, x = blockIdx.x;
    if ((G & 7) == 0) {
      const int X = x & 7;
      first = static_cast<int>((static_cast<long long>(n_units) * X) >> 3) + (x >> 3);
      end = static_cast<int>((static_cast<long long>(n_units) * (X + 1)) >> 3);
      stride = G >> 3;
    } else {
      first = x;
      end = n_units;
      stride = G;
    }
  }
  if (first >= end) return;

  Cursor cur = cursor_at<T, BS, kind>(kargs(), first);
  Unit cu = decode_unit<T, BS, kind>(kargs(), cur);
  u32x4 qop[C::QC];
  {
    const kargs_ptr a = kargs();
    issue_tile<T, BS, 0>((gchar_ptr)(a->k) + cu.off, (gchar_ptr)(a->v) + cu.off, tile_at(cu.tl, 0), wave, lane);
    load_q<T, BS>(a->q + cu.off + static_cast<size_t>(cu.q0) * C::ROWB, wq, lane, qop);
  }
  for (;;) {
    // Per-lane address arithmetic is redone for every unit rather than kept
    // live across the unit loop (register pressure).
    // (The lane id is rebuilt from the exec mask for every unit, by asm the
    // compiler cannot hoist, rather than kept in a register: kept, it was
    // spilled, and reloading it drained the prefetch.)
    const int lane_u = lane_id_here();
    const Cursor nxt = cursor_advance<T, BS, kind>(kargs(), cur, stride);
    const bool has_next = nxt.unit < end;
    NextUnit nx;
    {
      const Unit nu = decode_unit<T, BS, kind>(kargs(), nxt);
      nx.off = nu.off;
      nx.q0 = nu.q0;
      if constexpr (kind == 3)   // a chunk may start at a random block: read the table only
        nx.tile0 = has_next ? tile_at(nu.tl, 0) : 0;   // for a unit that exists
      else
        nx.tile0 = nu.tl.global ? nu.tl.first : 0;
      nx.pf = has_next && (cu.ntiles & 1) == 0 ? 1 : 0;
      nx.unused = 0;
    }
    gchar_ptr kbh, vbh;
    const uint8_t* pad_b;
    {
      const kargs_ptr a = kargs();
      kbh = (gchar_ptr)(a->k) + cu.off;
      vbh = (gchar_ptr)(a->v) + cu.off;
      pad_b = HAS_PAD ? a->pad + static_cast<size_t>(cu.b) * a->L : nullptr;
    }
    const int ntiles = cu.ntiles;

    WaveState ws;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      ws.o[0][v] = 0.0f;
      ws.o[1][v] = 0.0f;
    }
    ws.m = -__builtin_inff();
    ws.l = 0.0f;
    ws.qs = 1.0f;
    ws.big = 0.0f;
    if constexpr (HAS_PAD) {
      if (kargs()->qmask) ws.qs = pad_b[cu.q0 + wq * 32 + (lane_u & 31)] != 0 ? 1.0f : 0.0f;
    }

    // ---- tile loop: trips of 8 straight-line steps ----------------------------
    // Middle units at r <= 3 and the global chunks have at most 8 tiles, so
    // one trip covers them; longer lists take more.  Tile ids are computed
    // once per trip, one list position per lane (tile_ids()): the trip's and
    // the one after it (its last step prefetches that tile), then read out of
    // their lanes two per scalar register (nb < 65536), so that no vector
    // register holds them across the trip.
    // (Trips of 12 were 1% slower at r = 3.)
    constexpr int TRIP = 8;
    static_assert(TRIP % 2 == 0, "trip must keep the stage parity aligned");
    for (int u = 0; u < ntiles; u += TRIP) {
      // Tiles left from u.  Opaque, so that the step guards and the last-step
      // test compare it with immediates rather than with one precomputed
      // ntiles - k per step (scalar registers that would spill).
      int rem = ntiles - u;
      asm volatile("" : "+s"(rem));
      uint32_t tp[(TRIP + 2) / 2];
      {
        const int tv = tile_ids(cu.tl, u, lane_u);
#pragma unroll
        for (int k = 0; k < (TRIP + 2) / 2; ++k)
          tp[k] = static_cast<uint32_t>(__builtin_amdgcn_readlane(tv, 2 * k)) |
                  (static_cast<uint32_t>(__builtin_amdgcn_readlane(tv, 2 * k + 1)) << 16);
      }
#define BB_TILE(k) static_cast<int>((tp[(k) >> 1] >> (16 * ((k) & 1))) & 0xffffu)
#define BB_STEP(k)                                                                                  \
  if ((k) < rem)                                                                                    \
    step<T, BS, (k) % 2, HAS_PAD>(ws, qop, u + (k) == 0, (k) + 1 == rem, BB_TILE(k), BB_TILE((k) + 1),  \
                                  kbh, vbh, pad_b, wave, lane_u, kbase, nx, wq);
      BB_STEP(0) BB_STEP(1) BB_STEP(2) BB_STEP(3) BB_STEP(4) BB_STEP(5)
      BB_STEP(6) BB_STEP(7)
#undef BB_STEP
#undef BB_TILE
    }

    if constexpr (sizeof(T) == 2) {
      // a probability above the fixed reference's bound: this wave's keys of
      // the unit again, exactly (rare; see softmax_pv)
      if (__any(ws.big > kProbBound)) redo_unit_w<1, HAS_PAD, 1>(ws, cu, ntiles, wq, lane_u, kbase);
    }
    if ((ntiles - 1) & 1)
      finalize<T, BS, 1>(ws, cu, wq, wk, lane_u);
    else
      finalize<T, BS, 0>(ws, cu, wq, wk, lane_u);
    if (!has_next) break;
    if (!nx.pf) {
      // odd tile count: the merge went through stage 0, which the next unit's
      // first tile now refills once every wave is past the merge
      lds_barrier();
      const kargs_ptr a = kargs();
      issue_tile<T, BS, 0>((gchar_ptr)(a->k) + nx.off, (gchar_ptr)(a->v) + nx.off, nx.tile0, wave, lane_u);
      load_q<T, BS>(a->q + nx.off + static_cast<size_t>(nx.q0) * C::ROWB, wq, lane_u, qop);
    }
    cur = nxt;
    cu = decode_unit<T, BS, kind>(kargs(), cur);
  }
}

// Split-K merge of the two global query blocks of one (b, h): the partials of
// the n_s key chunks (row max m_s, row sum l_s, unnormalised O_s) combine as
// out = sum_s 2^((m_s - m)c) O_s / sum_s 2^((m_s - m)c) l_s, m = max_s m_s.
// Runs as its own launch after the global-row units, so their partials are
// complete and visible without any in-kernel fence.  A workgroup covers 8
// rows of one query group of one 64-row unit block, all 64 dims: thread
// (cs, q, g, jj) takes the 4-dim groups (keep 0 and 1, q) of row 8 rb + jj
// for lane half g (so each chunk's loads are 128-byte runs of the partial
// layout), over the chunks s = cs, cs + kMergeSplit, ... in one online pass;
// the kMergeSplit chunk groups are then combined through LDS in a fixed
// order, so the result is deterministic.
constexpr int kMergeSplit = 4;

// ALL = false: the two global blocks of every (b, h), n_s chunks each.  ALL =
// true (after kind 3 units): every query block, gc chunks for the global
// blocks and mc for the middle ones (slot order of decode_unit).
template <typename T, int BS, bool ALL>
__global__ void __launch_bounds__(64 * kMergeSplit) bb_global_merge_kernel(Args a) {
  constexpr int ROWB = kD * sizeof(T);
  constexpr int UB = BS / 64;                                 // 64-row unit blocks per query block
  __shared__ float s_m[kMergeSplit][64], s_l[kMergeSplit][64];
  __shared__ f32x4 s_o[kMergeSplit][2][64];
  const int rb = blockIdx.x & 3;                              // 8-row slice of the query group
  const int wq = (blockIdx.x >> 2) & 1;
  const int rest = blockIdx.x >> 3;
  const int qh = rest % UB, gblk = rest / UB;
  int bh, qb, n_ch;
  size_t base;
  if constexpr (ALL) {
    bh = gblk / a.nb;
    qb = gblk - bh * a.nb;
    const size_t slots = static_cast<size_t>(2 * a.gc + (a.nb - 2) * a.mc);
    const int first = qb == 0 ? 0 : (qb == a.nb - 1 ? a.gc : 2 * a.gc + (qb - 1) * a.mc);
    n_ch = qb == 0 || qb == a.nb - 1 ? a.gc : a.mc;
    base = static_cast<size_t>(bh) * slots + first;
  } else {
    bh = gblk >> 1;
    const int gsel = gblk & 1;
    qb = gsel ? a.nb - 1 : 0;
    n_ch = a.n_s;
    base = (static_cast<size_t>(bh) * 2 + gsel) * a.n_s;
  }
  const int cs = threadIdx.x >> 6, t = threadIdx.x & 63;
  const int q = t >> 4, g = (t >> 3) & 1, j = rb * 8 + (t & 7);
  const int lane = j + 32 * g;
  const int row = qh * 64 + wq * 32 + j;                      // row inside the query block
  float m = -__builtin_inff();
  float den = 0.0f;
  f32x4 num[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll 2
  for (int s = cs; s < n_ch; s += kMergeSplit) {
    const size_t pi = (base + s) * BS + row;
    const float* blk = a.po + ((base + s) * BS + qh * 64) * kD;
    const float ms = a.pm[pi], ls = a.pl[pi];
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(blk + partial_slot(wq, 0, q, lane));
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(blk + partial_slot(wq, 1, q, lane));
    const float mn = fmaxf(m, ms);
    const float c0 = __builtin_amdgcn_exp2f((m - mn) * kScaleLog2);   // 0 while m is -inf
    const float c1 = __builtin_amdgcn_exp2f((ms - mn) * kScaleLog2);
    den = den * c0 + ls * c1;
    num[0] = num[0] * c0 + o0 * c1;
    num[1] = num[1] * c0 + o1 * c1;
    m = mn;
  }
  s_m[cs][t] = m;
  s_l[cs][t] = den;
  s_o[cs][0][t] = num[0];
  s_o[cs][1][t] = num[1];
  __syncthreads();
  if (cs != 0) return;
  float mm = s_m[0][t];
#pragma unroll
  for (int c = 1; c < kMergeSplit; ++c) mm = fmaxf(mm, s_m[c][t]);
  float dd = 0.0f;
  f32x4 nn[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
  for (int c = 0; c < kMergeSplit; ++c) {
    if (s_m[c][t] == -__builtin_inff()) continue;             // group had no chunk
    const float w = __builtin_amdgcn_exp2f((s_m[c][t] - mm) * kScaleLog2);
    dd += w * s_l[c][t];
    nn[0] += w * s_o[c][0][t];
    nn[1] += w * s_o[c][1][t];
  }
  const float inv = __builtin_amdgcn_rcpf(dd);
  char* orow = a.out + (static_cast<size_t>(bh) * a.L + static_cast<size_t>(qb) * BS + row) * ROWB;
  if (a.lse != nullptr && q == 0 && g == 0)
    a.lse[static_cast<size_t>(bh) * a.L + static_cast<size_t>(qb) * BS + row] =
        (mm * kScaleLog2 + __builtin_amdgcn_logf(dd)) * kLn2;
#pragma unroll
  for (int keep = 0; keep < 2; ++keep) {
    const int d0 = 32 * keep + 16 * (q >> 1) + 8 * g + 4 * (q & 1);
    store_f32x4(orow + d0 * sizeof(T), nn[keep] * inv, static_cast<T*>(nullptr));
  }
}

template <typename T, int BS, bool HAS_PAD>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) __attribute__((amdgpu_waves_per_eu(4))) bb_fused_kernel(Args, int n_units) {
  run<T, BS, 0, HAS_PAD>(n_units);
}
template <typename T, int BS, bool HAS_PAD>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) __attribute__((amdgpu_waves_per_eu(4))) bb_global_rows_kernel(Args, int n_units) {
  run<T, BS, 1, HAS_PAD>(n_units);
}
template <typename T, int BS, bool HAS_PAD>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) __attribute__((amdgpu_waves_per_eu(4))) bb_middle_rows_kernel(Args, int n_units) {
  run<T, BS, 2, HAS_PAD>(n_units);
}
template <typename T, int BS, bool HAS_PAD>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) __attribute__((amdgpu_waves_per_eu(4))) bb_small_kernel(Args, int n_units) {
  run<T, BS, 3, HAS_PAD>(n_units);
}

// ============================================ forward, bf16, block 128 ==
// The bf16 work-unit kernel for block 128.  The work units (64 query rows of
// a block; a key block streams as two 64-key tiles, b -> 2b and 2b+1),
// tile lists, operand layouts and split-K partials are those of run() above;
// what differs is the shape of the work per wave and the softmax:
//   - a workgroup is 2 waves, the two 32-row query groups of a 64-row unit,
//     and each wave owns complete query rows: every step covers one 32-key
//     subtile with both waves, so a unit ends without any merge between
//     waves (for block 128, run() merges four key groups in two LDS rounds);
//   - a ring stage holds one 32-key subtile of K and of V (8 KiB), so a
//     workgroup needs 16 KiB of LDS and a CU holds 8 of them: 4 waves per
//     SIMD at up to 128 registers each;
//   - the softmax takes every probability of a row in a unit against one
//     fixed reference (below), with no rescale branch in the step.
//
// Softmax with a fixed reference.  Within a unit, each row's probabilities
// are taken against one reference m: the row max of the unit's first 32-key
// subtile (pad offsets included).  m is a score of the row, so the largest
// probability of the row is at least 1 (no underflow of the dominant terms).
// Each subtile checks that its probabilities stay bounded: the lane's sum of
// them (computed anyway for the row sum) must not exceed 2^32, so no single
// one does; then O and l are far inside fp32 range and need no rescaling.
// When some lane's sum exceeds the bound (scores more than 32/c above m, or
// an all-padding first subtile against valid later ones), that wave
// recomputes its rows of the unit at the end, exactly, in two passes from
// global memory (redo_unit_w).

// End of a unit: each wave holds complete rows.  Middle unit: out = O / l in
// bf16 (and the row log-sum-exp when asked for); global unit: the
// unnormalised partial (max, sum, O) in the layout of partial_slot().
__device__ __forceinline__ void finalize_w(const WaveStateW& ws, const Unit& w, int wq, int lane) {
  const int j = lane & 31, g = lane >> 5;
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ws.l), __float_as_uint(ws.l), false, false);
  const float l = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);   // both lane halves of the row
  if (w.gsel < 0) {
    const float inv = __builtin_amdgcn_rcpf(l);
    char* dst = kargs()->out + w.off + static_cast<size_t>(w.q0 + wq * 32 + j) * (kD * 2);
    float* lse = kargs()->lse;
    if (g == 0 && lse != nullptr)
      lse[w.off / (kD * 2) + w.q0 + wq * 32 + j] = (ws.m * kScaleLog2 + __builtin_amdgcn_logf(l)) * kLn2;
#pragma unroll
    for (int keep = 0; keep < 2; ++keep)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ws.o[keep][8 * h8 + e] * inv;
        store_row8(dst + (keep * 32 + 16 * h8 + 8 * g) * 2, x, static_cast<__bf16*>(nullptr));
      }
    return;
  }
  const kargs_ptr a = kargs();
  const size_t pidx = w.pbase + wq * 32 + j;
  float* blk = a->po + w.pbase * kD;
#pragma unroll
  for (int keep = 0; keep < 2; ++keep)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v4 = {ws.o[keep][4 * q], ws.o[keep][4 * q + 1], ws.o[keep][4 * q + 2], ws.o[keep][4 * q + 3]};
      *reinterpret_cast<f32x4*>(blk + partial_slot(wq, keep, q, lane)) = v4;
    }
  if (g == 0) {
    a->pm[pidx] = ws.m;
    a->pl[pidx] = l;
  }
}

// The 32-key-step kernel: its ring, step and persistent workgroup.  A
// unit's subtile count is even, so its last step always sits in stage 1 and
// the next unit's first subtile and Q rows are always prefetched during it.

constexpr int kSub32NW = 2;                   // waves per workgroup
constexpr int kSub32NT = 64 * kSub32NW;
constexpr int kSub = 32 * kD * 2;              // one 32-key bf16 subtile of K (or V): 4 KiB

// The 2-stage ring of 32-key stages (K subtile, then V subtile).
template <int S>
struct SubStage {
  static __device__ __forceinline__ char* buf() {
    __shared__ __attribute__((aligned(1024))) char b[2 * kSub];
    return b;
  }
  static __device__ __forceinline__ char* k() { return buf(); }
  static __device__ __forceinline__ char* v() { return buf() + kSub; }
};

// DMA of 32-key subtile `sub` (keys [32 sub, 32 sub + 32)) of K and V into
// stage S: 4 instructions per matrix, 2 per wave; the swizzled chunk
// placement of issue_tile().
template <int S>
__device__ __forceinline__ void issue_sub(gchar_ptr kbh, gchar_ptr vbh, int sub, int wave, int lane) {
  constexpr int CPR = kD * 2 / 16;
  const gchar_ptr kt = kbh + static_cast<size_t>(sub) * kSub;
  const gchar_ptr vt = vbh + static_cast<size_t>(sub) * kSub;
  const uint32_t lk = lds_addr(SubStage<S>::k()), lv = lk + kSub;
  uint32_t ko[2], vo[2], mk[2], mv[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int ins = wave + kSub32NW * jj;
    const int slot = ins * 64 + lane;
    const int row = slot / CPR, p = slot % CPR;
    ko[jj] = row * (kD * 2) + ((p ^ swz_k(row)) << 4);
    vo[jj] = row * (kD * 2) + ((p ^ swz_v(row)) << 4);
    mk[jj] = __builtin_amdgcn_readfirstlane(lk + ins * 1024);
    mv[jj] = __builtin_amdgcn_readfirstlane(lv + ins * 1024);
  }
  dma16x4(kt, vt, ko[0], vo[0], ko[1], vo[1], mk[0], mv[0], mk[1], mv[1]);
}

// S^T = K . Q^T for the 32-key subtile in stage S (K rows perm_row-ordered
// as in scores()).
template <int S>
__device__ __forceinline__ f32x16 scores_n(const u32x4 (&qop)[4], int lane) {
  const int j = lane & 31, g = lane >> 5;
  const char* sk = SubStage<S>::k();
  const int row = perm_row(j);
  const int sw = swz_k(row);
  u32x4 a[4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
    a[x] = *reinterpret_cast<const u32x4*>(sk + row * (kD * 2) + (((2 * x + g) ^ sw) << 4));
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x) acc = mfma_qk(a[x], qop[x], acc, static_cast<__bf16*>(nullptr));
  return acc;
}

// V^T operands of the subtile in stage S (the transposing reads of load_v()).
template <int S>
__device__ __forceinline__ VOp<__bf16> load_v_n(int lane) {
  const char* sv = SubStage<S>::v();
  VOp<__bf16> vo;
  const int g = lane >> 5, e4 = (lane >> 2) & 3;
  const int r0 = 8 * g + e4;
#pragma unroll
  for (int dh = 0; dh < 2; ++dh) {
    const int dstart = dh * 32 + perm_row(16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    const int dchunk = dstart >> 3, dbyte = (dstart & 7) * 2;
    const char* base = sv + r0 * (kD * 2) + ((dchunk ^ swz_v(r0)) << 4) + dbyte;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + 16 * mm * (kD * 2)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + (16 * mm + 4) * (kD * 2)));
      vo.a[dh][mm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  return vo;
}

// Step i of a unit's subtile loop: subtile i sits in stage S = i % 2; sub_u
// and sub_fill are the ids of subtiles i and i+1.  FIRST: the unit's first
// subtile, whose row max is the reference.  On the last step (always in
// stage 1) the next unit's first subtile and Q rows are prefetched.
template <int S, bool HAS_PAD, bool FIRST>
__device__ __forceinline__ void step_n(WaveStateW& ws, u32x4 (&qop)[4], bool last, int sub_u, int sub_fill,
                                       gchar_ptr kbh, gchar_ptr vbh, const uint8_t* pad_b, int wave, int lane,
                                       const NextUnit& nx) {
  // The pad bytes first, so that their scalar load completes under the wait
  // and the barrier (see step()).
  PadWords pw;
  if constexpr (HAS_PAD) {
    pw = load_pad(pad_b + static_cast<size_t>(sub_u) * 32, 0);
    asm volatile("" ::: "memory");
  }
  __builtin_amdgcn_s_waitcnt(7 << 4);
  ring_barrier();
  f32x16 s = scores_n<S>(qop, lane);
  const VOp<__bf16> vo = load_v_n<S>(lane);
  if (!last) {
    issue_sub<S ^ 1>(kbh, vbh, sub_fill, wave, lane);
  } else if (S == 1 && nx.pf) {
    const kargs_ptr a = kargs();
    issue_sub<0>((gchar_ptr)(a->k) + nx.off, (gchar_ptr)(a->v) + nx.off, nx.tile0, wave, lane);
  }
  PadClass c;
  c.bias = 0.0f;
  c.mixed = 0u;
  if constexpr (HAS_PAD) {
    c = classify_pad(pw);
    if (c.mixed) add_pad_bias(s, c.mixed, lane, ws.qs);
    c.bias *= ws.qs;
  }
  if (S == 1 && last && nx.pf) {
    // Q is dead after the score products: refill it for the next unit
    asm volatile("" : "+v"(s) : : "memory");
    load_q<__bf16, 64>(kargs()->q + nx.off + static_cast<size_t>(nx.q0) * (kD * 2), wave, lane, qop);
  }
  if constexpr (FIRST) {
    const float lm = lane_max(s, s[15]) + c.bias;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lm), __float_as_uint(lm), false, false);
    ws.m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  bf16x8 pb[2];
  const float lsum = probs_w(s, ws.m, c.bias, pb);
  ws.l += lsum;
  ws.big = fmaxf(ws.big, lsum);
  pv_w(ws, vo, pb);
}

// The persistent workgroup of the 32-key-step kernel: run() above with its
// steps (and no merge between waves).
template <int BS, int kind, bool HAS_PAD>
__device__ __forceinline__ void run_n(int n_units) {
  constexpr int TPB = BS / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int first, stride, end;
  {
    const int G = gridDim.x, x = blockIdx.x;
    if ((G & 7) == 0) {
      const int X = x & 7;
      first = static_cast<int>((static_cast<long long>(n_units) * X) >> 3) + (x >> 3);
      end = static_cast<int>((static_cast<long long>(n_units) * (X + 1)) >> 3);
      stride = G >> 3;
    } else {
      first = x;
      end = n_units;
      stride = G;
    }
  }
  if (first >= end) return;

  Cursor cur = cursor_at<__bf16, BS, kind>(kargs(), first);
  Unit cu = decode_unit<__bf16, BS, kind>(kargs(), cur);
  u32x4 qop[4];
  {
    const kargs_ptr a = kargs();
    issue_sub<0>((gchar_ptr)(a->k) + cu.off, (gchar_ptr)(a->v) + cu.off, 2 * tile64_at<TPB>(cu.tl, 0), wave, lane);
    load_q<__bf16, 64>(a->q + cu.off + static_cast<size_t>(cu.q0) * (kD * 2), wave, lane, qop);
  }
  for (;;) {
    int lane_u = static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
    asm volatile("" : "+v"(lane_u));
    const Cursor nxt = cursor_advance<__bf16, BS, kind>(kargs(), cur, stride);
    const bool has_next = nxt.unit < end;
    const int ntiles = TPB * cu.ntiles;        // 64-key tiles
    const int nsub = 2 * ntiles;               // 32-key steps (even)
    NextUnit nx;
    {
      const Unit nu = decode_unit<__bf16, BS, kind>(kargs(), nxt);
      nx.off = nu.off;
      nx.q0 = nu.q0;
      nx.tile0 = 2 * TPB * (nu.tl.global ? nu.tl.first : 0);   // its first 32-key subtile
      nx.pf = has_next ? 1 : 0;
      nx.unused = 0;
    }
    gchar_ptr kbh, vbh;
    const uint8_t* pad_b;
    {
      const kargs_ptr a = kargs();
      kbh = (gchar_ptr)(a->k) + cu.off;
      vbh = (gchar_ptr)(a->v) + cu.off;
      pad_b = HAS_PAD ? a->pad + static_cast<size_t>(cu.b) * a->L : nullptr;
    }
    WaveStateW ws;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      ws.o[0][v] = 0.0f;
      ws.o[1][v] = 0.0f;
    }
    ws.m = -__builtin_inff();
    ws.l = 0.0f;
    ws.big = 0.0f;
    ws.qs = 1.0f;
    if constexpr (HAS_PAD) {
      if (kargs()->qmask) ws.qs = pad_b[cu.q0 + wave * 32 + (lane_u & 31)] != 0 ? 1.0f : 0.0f;
    }

    // trips of TRIP straight-line steps (TRIP / 2 tiles).  Longer trips mean
    // fewer tile-id computations per unit (a unit at r = 4 runs 36 steps);
    // the lengths kept measured fastest: 16 without padding (2.5% faster than
    // 8 on 1 x 12 x 32768), 12 with it (1.2%; 16 spilled more there).
    constexpr int TRIP = HAS_PAD ? 12 : 16;
    static_assert(TRIP % 4 == 0 && TRIP <= 16, "trip must keep the stage parity aligned");
    for (int u = 0; u < nsub; u += TRIP) {
      int rem = nsub - u;
      asm volatile("" : "+s"(rem));
      // the trip's 64-key tiles and the one after it, two 16-bit ids per
      // scalar register (L / 64 < 65536)
      const int t0 = u >> 1, tleft = ntiles - t0;
      uint32_t tp[(TRIP / 2 + 2) / 2];
#pragma unroll
      for (int k = 0; k < (TRIP / 2 + 2) / 2; ++k) {
        const uint32_t ta = 2 * k < tleft ? static_cast<uint32_t>(tile64_at<TPB>(cu.tl, t0 + 2 * k)) : 0u;
        const uint32_t tb = 2 * k + 1 < tleft ? static_cast<uint32_t>(tile64_at<TPB>(cu.tl, t0 + 2 * k + 1)) : 0u;
        tp[k] = ta | (tb << 16);
      }
#define BB_SUB(k) (2 * static_cast<int>((tp[(k) >> 2] >> (16 * (((k) >> 1) & 1))) & 0xffffu) + ((k) & 1))
#define BB_STEPN(k, F)                                                                                           \
  step_n<(k) % 2, HAS_PAD, F>(ws, qop, (k) + 1 == rem, BB_SUB(k), BB_SUB((k) + 1), kbh, vbh, pad_b, wave, lane_u, \
                              nx)
      if (u == 0)
        BB_STEPN(0, true);
      else
        BB_STEPN(0, false);
#define BB_STEPN_IF(k) \
  if constexpr ((k) < TRIP) {            \
    if ((k) < rem) BB_STEPN(k, false);   \
  }
      BB_STEPN_IF(1) BB_STEPN_IF(2) BB_STEPN_IF(3) BB_STEPN_IF(4) BB_STEPN_IF(5) BB_STEPN_IF(6) BB_STEPN_IF(7)
      BB_STEPN_IF(8) BB_STEPN_IF(9) BB_STEPN_IF(10) BB_STEPN_IF(11) BB_STEPN_IF(12) BB_STEPN_IF(13)
      BB_STEPN_IF(14) BB_STEPN_IF(15)
#undef BB_STEPN_IF
#undef BB_STEPN
#undef BB_SUB
    }
    if (__any(ws.big > kProbBound)) redo_unit_w<TPB, HAS_PAD, 2>(ws, cu, ntiles, wave, lane_u, 0);
    finalize_w(ws, cu, wave, lane_u);
    if (!has_next) break;
    cur = nxt;
    cu = decode_unit<__bf16, BS, kind>(kargs(), cur);
  }
}

template <int BS, bool HAS_PAD>
__global__ void __launch_bounds__(kSub32NT) __attribute__((amdgpu_waves_per_eu(4))) bb_sub32_fused_kernel(Args, int n_units) {
  run_n<BS, 0, HAS_PAD>(n_units);
}
template <int BS, bool HAS_PAD>
__global__ void __launch_bounds__(kSub32NT) __attribute__((amdgpu_waves_per_eu(4))) bb_sub32_global_rows_kernel(Args, int n_units) {
  run_n<BS, 1, HAS_PAD>(n_units);
}
template <int BS, bool HAS_PAD>
__global__ void __launch_bounds__(kSub32NT) __attribute__((amdgpu_waves_per_eu(4))) bb_sub32_middle_rows_kernel(Args, int n_units) {
  run_n<BS, 2, HAS_PAD>(n_units);
}

// ================================================================ backward ==
// Gradients of the same attention (dQ, dK, dV of sum(out * dO)), the
// textbook softmax-attention backward restricted to the block pattern:
//   P = 2^(s c + bias c - LSE2) rebuilt from the forward's row log-sum-exp
//   (LSE2 = LSE log2(e), c = log2(e)/sqrt(d)), D_t = sum_d dO[t] O[t],
//   dS = P (dP - D) with dP = dO V^T,
//   dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d), dV = P^T dO.
// Two passes over the pattern plus a small reduce:
//   bb_bwd_dq_kernel     query-stationary (the forward's work units): D and
//                        LSE2 of its rows (stored for the next pass), then per
//                        key tile S^T = K Q^T, dP^T = V dO^T, dS^T,
//                        dQ^T += K^T dS^T; the two global query blocks as
//                        split-K chunks;
//   bb_bwd_dkdv_kernel   key-stationary: a middle key block j is seen by the
//                        global query blocks, the band rows {j-1, j, j+1} and
//                        the middle rows whose random list holds j (the
//                        inverted table); per query tile S = Q K^T, dP = dO V^T,
//                        dV^T += dO^T P, dK^T += Q^T dS; the two global key
//                        blocks (seen by every query block) as split-K chunks;
//   bb_bwd_reduce_kernel sums the split-K partials of those four blocks.
// Problems with too few units to fill the device run kind 3 units in both
// passes instead (bwd_split()): every query block's key tiles and every key
// block's query tiles cut into chunks, every chunk a partial, and the reduce
// sums the chunks of every block.
// Every pass stages its streamed tiles through the same two-stage LDS ring
// as the forward; a tile that is read both as rows and transposed is read
// one of the two ways through the other matrix's swizzle (correct, with
// some bank conflicts).

struct BwdArgs {
  Args f;                   // q, k, v, pad, rand_idx and the sizes (first member: kargs() reads it)
  const char* o;            // forward output O [B*H][L][d]
  const char* dout;         // dO [B*H][L][d]
  const float* lse;         // forward row log-sum-exp (natural log) [B*H][L]
  const int32_t* inv_off;   // [H][nb+1] ranges of inv_rows per (head, key block)
  const int32_t* inv_rows;  // middle query blocks holding each key block in their random list
  f32x2* rowstat;           // workspace [B*H][L]: (LSE * log2(e), D) per row
  float* dq_part;           // workspace [B*H][2][n_s][BS][d], lane-major 64 x 64 blocks
  float* dk_part;
  float* dv_part;
  char* dq;
  char* dk;
  char* dv;
};

typedef const __attribute__((address_space(4))) BwdArgs* bargs_ptr;
__device__ __forceinline__ bargs_ptr bargs() {
  bargs_ptr p = (bargs_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

// 32 rows of stage S's K slot (SLOT 0, K swizzle) or V slot (SLOT 1, V
// swizzle), permuted as in scores(), times the B operand bop: the 32 x 32
// product rows x bop-columns.
template <typename T, int BS, int S, int SLOT>
__device__ __forceinline__ f32x16 rows_times(const u32x4 (&bop)[Cfg<T, BS>::QC], int rbase, int lane) {
  using C = Cfg<T, BS>;
  const int j = lane & 31, g = lane >> 5;
  const char* sb = SLOT ? Stage<T, BS, S>::v() : Stage<T, BS, S>::k();
  const int row = rbase + perm_row(j);
  const int sw = SLOT ? swz_v(row) : swz_k(row);
  u32x4 a[C::QC];
#pragma unroll
  for (int x = 0; x < C::QC; ++x)
    a[x] = *reinterpret_cast<const u32x4*>(sb + row * C::ROWB + (((2 * x + g) ^ sw) << 4));
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int x = 0; x < C::QC; ++x) acc = mfma_qk(a[x], bop[x], acc, static_cast<T*>(nullptr));
  return acc;
}

// The transposed operand of 32 rows [rbase, rbase + 32) of a slot (the
// forward's load_v, for either slot and its swizzle; both swizzles keep rows
// r, r+4, r+16 and r+20 on one pattern).
template <typename T, int BS, int S, int SLOT>
__device__ __forceinline__ VOp<T> cols_op(int rbase, int lane) {
  using C = Cfg<T, BS>;
  const char* sb = SLOT ? Stage<T, BS, S>::v() : Stage<T, BS, S>::k();
  VOp<T> vo;
  if constexpr (sizeof(T) == 4) {
    // fp32 (32x32x2 products): lane (dim, g) takes row 16 (v / 8) + 8 g + v % 8
    // of the 32, one float per product, as the forward's fp32 V^T reads
    const int j = lane & 31, g = lane >> 5;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const int dim = dh * 32 + perm_row(j);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = rbase + 16 * (v >> 3) + 8 * g + (v & 7);
        const int sw = SLOT ? swz_v(row) : swz_k(row);
        vo.a[dh][v] = *reinterpret_cast<const float*>(sb + row * C::ROWB + (((dim >> 2) ^ sw) << 4) + (dim & 3) * 4);
      }
    }
    return vo;
  } else {
  const int g = lane >> 5, e4 = (lane >> 2) & 3;
  const int r0 = rbase + 8 * g + e4;
  const int sw = SLOT ? swz_v(r0) : swz_k(r0);
#pragma unroll
  for (int dh = 0; dh < 2; ++dh) {
    const int dstart = dh * 32 + perm_row(16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    const int dchunk = dstart >> 3, dbyte = (dstart & 7) * 2;
    const char* base = sb + r0 * C::ROWB + ((dchunk ^ sw) << 4) + dbyte;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + 16 * mm * C::ROWB));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + (16 * mm + 4) * C::ROWB));
      vo.a[dh][mm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  return vo;
  }
}

// Two bf16 pairs per 4 fp32 values, in the PV operand layout.
__device__ __forceinline__ void pack_pairs(const float (&x)[16], bf16x8 (&pb)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      f32x2 pr = {x[8 * h + e], x[8 * h + e + 1]};
      const bf16x2 c2 = __builtin_convertvector(pr, bf16x2);
      pb[h][e] = c2[0];
      pb[h][e + 1] = c2[1];
    }
}

// acc[dh] += A[dh] . X over this subtile's 32 rows, with A a transposed
// operand (cols_op) and X the 16 fp32 values of a score-type product (lane =
// column): bf16 pairs into 32x32x16 products, or fp32 into 32x32x2 ones.
__device__ __forceinline__ void tprod(f32x16 (&acc)[2], const VOp<__bf16>& a, const float (&x)[16]) {
  bf16x8 xb[2];
  pack_pairs(x, xb);
#pragma unroll
  for (int mm = 0; mm < 2; ++mm)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
      acc[dh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.a[dh][mm], xb[mm], acc[dh], 0, 0, 0);
}
__device__ __forceinline__ void tprod(f32x16 (&acc)[2], const VOp<float>& a, const float (&x)[16]) {
#pragma unroll
  for (int v = 0; v < 16; ++v)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
      acc[dh] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[dh][v], x[v], acc[dh], 0, 0, 0);
}

// ---- dQ pass ----------------------------------------------------------------
// Stage layout: V in the K slot (its rows feed dP^T = V dO^T), K in the V
// slot (its transposed operand feeds dQ^T += K^T dS^T; its rows, read
// through the V swizzle, feed S^T = K Q^T).
template <typename T, int BS, int S, bool HAS_PAD, bool QM>
__device__ __forceinline__ void step_dq(WaveState& ws, const u32x4 (&qop)[Cfg<T, BS>::QC],
                                        const u32x4 (&dop)[Cfg<T, BS>::QC], float lse2, float dsum, bool last,
                                        int tile_u, int tile_fill, gchar_ptr vbh, gchar_ptr kbh,
                                        const uint8_t* pad_b, int wave, int lane, int kbase) {
  PadWords pw;
  if constexpr (HAS_PAD) {
    pw = load_pad(pad_b + static_cast<size_t>(tile_u) * BS, kbase);
    asm volatile("" ::: "memory");
  }
  __builtin_amdgcn_s_waitcnt(7 << 4);
  ring_barrier();
  f32x16 s = rows_times<T, BS, S, 1>(qop, kbase, lane);    // S^T = K Q^T
  const f32x16 dp = rows_times<T, BS, S, 0>(dop, kbase, lane);   // dP^T = V dO^T
  const VOp<T> kt = cols_op<T, BS, S, 1>(kbase, lane);       // K^T
  if (!last) issue_tile<T, BS, S ^ 1>(vbh, kbh, tile_fill, wave, lane);
  float pbias = 0.0f;
  if constexpr (QM)
    pbias = apply_pad(s, pw, lane, ws.qs) * ws.qs;
  else if constexpr (HAS_PAD)
    pbias = apply_pad(s, pw, lane);
  const float off = lse2 - pbias * kScaleLog2;
  float ds[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], kScaleLog2, -off));
    ds[v] = p * (dp[v] - dsum);
  }
  tprod(ws.o, kt, ds);
}

// Sum of the two key groups' dQ^T halves (exchanged through stage S), scaled
// by 1/sqrt(d); a middle unit writes its rows, a global unit its partial.
template <typename T, int BS, int S, int KEEP>
__device__ __forceinline__ void finalize_dq_half(WaveState& ws, const Unit& w, int wq, int lane) {
  using C = Cfg<T, BS>;
  constexpr int GIVE = KEEP ^ 1;
  float* mo0 = reinterpret_cast<float*>(Stage<T, BS, S>::k());
  float* mo1 = reinterpret_cast<float*>(Stage<T, BS, S>::v());
  float* mo_give = GIVE ? mo1 : mo0;
  const float* mo_keep = KEEP ? mo1 : mo0;
#pragma unroll
  for (int v = 0; v < 16; ++v) mo_give[(wq * 16 + v) * 64 + lane] = ws.o[GIVE][v];
  lds_barrier();
  const int j = lane & 31, g = lane >> 5;
  float x[2][8];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[h8][e] = ws.o[KEEP][8 * h8 + e] + mo_keep[(wq * 16 + 8 * h8 + e) * 64 + lane];
  const bargs_ptr b = bargs();
  if (w.gsel < 0) {
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[h8][e] *= 0.125f;   // 1/sqrt(64)
    char* dst = b->dq + w.off + static_cast<size_t>(w.q0 + wq * 32 + j) * C::ROWB;
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
      store_row8(dst + (KEEP * 32 + 16 * h8 + 8 * g) * C::ES, x[h8], static_cast<T*>(nullptr));
    return;
  }
  float* blk = b->dq_part + w.pbase * kD;
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 v4 = {x[h8][4 * hf], x[h8][4 * hf + 1], x[h8][4 * hf + 2], x[h8][4 * hf + 3]};
      *reinterpret_cast<f32x4*>(blk + partial_slot(wq, KEEP, 2 * h8 + hf, lane)) = v4;
    }
}

// End of a dQ unit: the key groups' dQ^T summed through stage S -- for four
// key groups (block 128) first 2,3 -> 0,1 in full, then 0 <-> 1 by head dims.
template <typename T, int BS, int S>
__device__ __forceinline__ void finalize_dq(WaveState& ws, const Unit& w, int wq, int wk, int lane) {
  using C = Cfg<T, BS>;
  float* mo0 = reinterpret_cast<float*>(Stage<T, BS, S>::k());
  float* mo1 = reinterpret_cast<float*>(Stage<T, BS, S>::v());
  lds_barrier();   // every wave is past its last LDS read of the unit
  if constexpr (C::WK == 4) {
    if (wk >= 2) {
      const int slot = (wk - 2) * C::WQ + wq;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        mo0[(slot * 16 + v) * 64 + lane] = ws.o[0][v];
        mo1[(slot * 16 + v) * 64 + lane] = ws.o[1][v];
      }
    }
    lds_barrier();
    if (wk < 2) {
      const int slot = wk * C::WQ + wq;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        ws.o[0][v] += mo0[(slot * 16 + v) * 64 + lane];
        ws.o[1][v] += mo1[(slot * 16 + v) * 64 + lane];
      }
    }
    lds_barrier();
  }
  if (wk == 0)
    finalize_dq_half<T, BS, S, 0>(ws, w, wq, lane);
  else if (wk == 1)
    finalize_dq_half<T, BS, S, 1>(ws, w, wq, lane);
  else
    lds_barrier();   // key groups 2 and 3: the last round's barrier
}

// KIND 0: the forward's ordinary units (middle query blocks finalised in
// place, global ones as split-K partials); KIND 3: the forward's small-problem
// units, every one a partial.
template <typename T, int BS, bool HAS_PAD, bool QM, int KIND>
__device__ __forceinline__ void run_dq(int n_units) {
  using C = Cfg<T, BS>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave % C::WQ, wk = wave / C::WQ;
  const int kbase = wk * 32;
  int first, stride, end;
  {
    const int G = gridDim.x, x = blockIdx.x;
    if ((G & 7) == 0) {
      const int X = x & 7;
      first = static_cast<int>((static_cast<long long>(n_units) * X) >> 3) + (x >> 3);
      end = static_cast<int>((static_cast<long long>(n_units) * (X + 1)) >> 3);
      stride = G >> 3;
    } else {
      first = x;
      end = n_units;
      stride = G;
    }
  }
  if (first >= end) return;
  Cursor cur = cursor_at<T, BS, KIND>(kargs(), first);
  for (;;) {
    const Unit cu = decode_unit<T, BS, KIND>(kargs(), cur);
    const bargs_ptr b = bargs();
    const size_t row = cu.off / C::ROWB + cu.q0 + wq * 32 + (lane & 31);
    u32x4 qop[C::QC], dop[C::QC], oop[C::QC];
    load_q<T, BS>(b->f.q + cu.off + static_cast<size_t>(cu.q0) * C::ROWB, wq, lane, qop);
    load_q<T, BS>(b->dout + cu.off + static_cast<size_t>(cu.q0) * C::ROWB, wq, lane, dop);
    load_q<T, BS>(b->o + cu.off + static_cast<size_t>(cu.q0) * C::ROWB, wq, lane, oop);
    // D = dO . O of this lane's row: each lane half holds half of the row's
    // chunks; the partner half adds the other.  LSE2 = LSE log2(e).  Both are
    // also stored for the dK/dV pass (by key group 0; global rows once per
    // split-K chunk, the same values).
    float dpart = 0.0f;
#pragma unroll
    for (int x = 0; x < C::QC; ++x) {
      if constexpr (sizeof(T) == 2) {
        const bf16x8 g8 = __builtin_bit_cast(bf16x8, dop[x]), o8 = __builtin_bit_cast(bf16x8, oop[x]);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart += static_cast<float>(g8[e]) * static_cast<float>(o8[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) dpart += __uint_as_float(dop[x][e]) * __uint_as_float(oop[x][e]);
      }
    }
    const auto dsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dpart), __float_as_uint(dpart), false, false);
    const float dsum = __uint_as_float(dsw[0]) + __uint_as_float(dsw[1]);
    const float lse2 = b->lse[row] * 1.4426950408889634f;
    if (wk == 0 && lane < 32) {
      const f32x2 rs = {lse2, dsum};
      b->rowstat[row] = rs;
    }
    const gchar_ptr vbh = (gchar_ptr)(b->f.v) + cu.off, kbh = (gchar_ptr)(b->f.k) + cu.off;
    const uint8_t* pad_b = HAS_PAD ? b->f.pad + static_cast<size_t>(cu.b) * b->f.L : nullptr;
    issue_tile<T, BS, 0>(vbh, kbh, tile_at(cu.tl, 0), wave, lane);
    WaveState ws;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      ws.o[0][v] = 0.0f;
      ws.o[1][v] = 0.0f;
    }
    ws.m = 0.0f;
    ws.l = 0.0f;
    // pair masking: a padded query row takes no key offsets (its uniform
    // offset cancels; the forward's log-sum-exp of such a row leaves it out)
    ws.qs = 1.0f;
    if constexpr (QM) ws.qs = pad_b[cu.q0 + wq * 32 + (lane & 31)] != 0 ? 1.0f : 0.0f;
    const int ntiles = cu.ntiles;
    constexpr int TRIP = 12;
    for (int u = 0; u < ntiles; u += TRIP) {
      int rem = ntiles - u;
      asm volatile("" : "+s"(rem));
      uint32_t tp[(TRIP + 2) / 2];
#pragma unroll
      for (int k = 0; k < (TRIP + 2) / 2; ++k) {
        const uint32_t t0 = 2 * k < rem ? static_cast<uint32_t>(tile_at(cu.tl, u + 2 * k)) : 0u;
        const uint32_t t1 = 2 * k + 1 < rem ? static_cast<uint32_t>(tile_at(cu.tl, u + 2 * k + 1)) : 0u;
        tp[k] = t0 | (t1 << 16);
      }
#define BB_TILE(k) static_cast<int>((tp[(k) >> 1] >> (16 * ((k) & 1))) & 0xffffu)
#define BB_STEP(k)                                                                                    \
  if ((k) < rem)                                                                                      \
    step_dq<T, BS, (k) % 2, HAS_PAD, QM>(ws, qop, dop, lse2, dsum, (k) + 1 == rem, BB_TILE(k),        \
                                     BB_TILE((k) + 1), vbh, kbh, pad_b, wave, lane, kbase);
      BB_STEP(0) BB_STEP(1) BB_STEP(2) BB_STEP(3) BB_STEP(4) BB_STEP(5)
      BB_STEP(6) BB_STEP(7) BB_STEP(8) BB_STEP(9) BB_STEP(10) BB_STEP(11)
#undef BB_STEP
#undef BB_TILE
    }
    if ((ntiles - 1) & 1)
      finalize_dq<T, BS, 1>(ws, cu, wq, wk, lane);
    else
      finalize_dq<T, BS, 0>(ws, cu, wq, wk, lane);
    lds_barrier();   // the exchange area is read before the next unit's first tile lands there
    cur = cursor_advance<T, BS, KIND>(kargs(), cur, stride);
    if (cur.unit >= end) break;
  }
}

// ---- dK/dV pass ---------------------------------------------------------------
// Work units per (b, h): the two global key blocks in n_s query chunks each
// (partials), then the nb-2 middle key blocks.  Query tiles of a middle key
// block j: 0, nb-1, the band rows max(1, j-1)..min(nb-2, j+1), then the rows
// of the inverted random table.  Stage layout: Q in the K slot, dO in the V slot.
struct KvTiles {
  int first;             // global key unit: first query tile of its chunk; middle: band start
  int nwin;              // middle: band rows inside 1..nb-2
  int nb;
  int global;
  int skip;              // middle unit: position of its first tile in the block's list
                         // (non-zero only for the query chunks of kind 3 units)
  int unused;            // (keeps the struct free of padding)
  const_i32_ptr inv;     // middle: its inverted-table rows
};

__device__ __forceinline__ int kv_tile_at(const KvTiles& tl, int u) {
  if (tl.global) return tl.first + u;
  u += tl.skip;
  if (u == 0) return 0;
  if (u == 1) return tl.nb - 1;
  if (u < 2 + tl.nwin) return tl.first + u - 2;
  const int e = tl.inv[u - 2 - tl.nwin];
  return e < 1 ? 1 : (e > tl.nb - 2 ? tl.nb - 2 : e);   // never read outside the sequence
}

struct KvUnit {
  size_t off;            // (b, h) byte offset
  size_t pbase;          // global key unit: partial row index of its first key row
  size_t bh;
  int b, k0, gsel, ntiles;
  KvTiles tl;
};

// Query tiles [i0, i1) of inv_rows seeing key block j of head h: the
// inverted table's range, clamped into the table, so that a corrupted offset
// cannot read outside it.
__device__ __forceinline__ void inv_range(bargs_ptr a, int h, int j, int& i0, int& i1) {
  const int nb = a->f.nb;
  const int32_t* offs = a->inv_off + static_cast<size_t>(h) * (nb + 1);
  const int total = a->f.H * (nb - 2) * a->f.r;
  const int o0 = offs[j], o1 = offs[j + 1];
  i0 = o0 < 0 ? 0 : (o0 > total ? total : o0);
  i1 = o1 < i0 ? i0 : (o1 > total ? total : o1);
}

// KIND 0: the ordinary units above.  KIND 3 (problems with too few units to
// fill the chip): every key block's query list split into chunks -- a->f.gc
// per global key block, a->f.mc per middle one, each a contiguous run of the
// list -- every unit writing partials, slots per (b, h) as for the dQ pass:
// [key block 0 chunks | key block nb-1 chunks | middle key block 1 chunks | ...].
template <typename T, int BS, int KIND>
__device__ __forceinline__ KvUnit decode_kv_unit(bargs_ptr a, const Cursor& c) {
  constexpr int KS = BS / 64;           // 64-key units per key block
  constexpr int LKS = KS == 2 ? 1 : 0;
  const int nb = a->f.nb, n_s = a->f.n_s;
  KvUnit w;
  w.bh = static_cast<size_t>(c.bh);
  w.off = static_cast<size_t>(c.bh) * a->f.L * Cfg<T, BS>::ROWB;
  w.b = c.b;
  w.tl.nb = nb;
  w.tl.skip = 0;
  w.tl.unused = 0;
  if constexpr (KIND == 3) {
    const int gc = a->f.gc, mc = a->f.mc;
    const size_t slots = static_cast<size_t>(2 * gc + (nb - 2) * mc);
    int slot, kb, kh;
    if (c.u < 2 * gc * KS) {
      const int half = gc * KS;
      w.gsel = c.u >= half ? 1 : 0;
      const int rem = c.u - (w.gsel ? half : 0);
      const int chunk = rem >> LKS;
      kh = rem & (KS - 1);
      kb = w.gsel ? nb - 1 : 0;
      slot = w.gsel * gc + chunk;
      w.tl.global = 1;
      w.tl.first = chunk * nb / gc;             // balanced chunks: none is empty (gc <= nb)
      w.ntiles = (chunk + 1) * nb / gc - w.tl.first;
      w.tl.nwin = 0;
      w.tl.inv = nullptr;
    } else {
      const int v = (c.u - 2 * gc * KS) >> LKS;
      kh = (c.u - 2 * gc * KS) & (KS - 1);
      const int mi = v / mc, chunk = v - mi * mc;
      kb = mi + 1;
      w.gsel = 2;
      slot = 2 * gc + mi * mc + chunk;
      const int lo = kb - 1 < 1 ? 1 : kb - 1;
      const int hi = kb + 1 > nb - 2 ? nb - 2 : kb + 1;
      int i0, i1;
      inv_range(a, c.h, kb, i0, i1);
      w.tl.global = 0;
      w.tl.first = lo;
      w.tl.nwin = hi - lo + 1;
      w.tl.inv = (const_i32_ptr)(a->inv_rows + i0);
      const int nt = 2 + w.tl.nwin + (i1 - i0);   // mc <= 2 + the fewest band rows: no chunk is empty
      w.tl.skip = chunk * nt / mc;
      w.ntiles = (chunk + 1) * nt / mc - w.tl.skip;
    }
    w.k0 = kb * BS + kh * 64;
    w.pbase = (static_cast<size_t>(c.bh) * slots + slot) * BS + kh * 64;
    return w;
  }
  const int n_g = 2 * n_s * KS;
  if (c.u < n_g) {
    w.gsel = c.u >= n_s * KS ? 1 : 0;
    const int rem = c.u - (w.gsel ? n_s * KS : 0);
    const int chunk = rem >> LKS, kh = rem & (KS - 1);
    w.k0 = (w.gsel ? nb - 1 : 0) * BS + kh * 64;
    w.pbase = ((static_cast<size_t>(c.bh) * 2 + w.gsel) * n_s + chunk) * BS + kh * 64;
    w.tl.global = 1;
    w.tl.first = chunk * kChunkTiles;
    w.tl.nwin = 0;
    w.tl.inv = nullptr;
    w.ntiles = nb - w.tl.first < kChunkTiles ? nb - w.tl.first : kChunkTiles;
  } else {
    w.gsel = -1;
    const int v = c.u - n_g;
    const int j = (v >> LKS) + 1, kh = v & (KS - 1);
    w.k0 = j * BS + kh * 64;
    w.pbase = 0;
    const int lo = j - 1 < 1 ? 1 : j - 1;
    const int hi = j + 1 > nb - 2 ? nb - 2 : j + 1;
    w.tl.global = 0;
    w.tl.first = lo;
    w.tl.nwin = hi - lo + 1;
    int i0, i1;
    inv_range(a, c.h, j, i0, i1);
    w.tl.inv = (const_i32_ptr)(a->inv_rows + i0);
    w.ntiles = 2 + w.tl.nwin + (i1 - i0);
  }
  return w;
}

struct KvState {
  f32x16 dk[2];   // dK^T, dims [0,32) and [32,64), 32 keys
  f32x16 dv[2];   // dV^T
};

// (LSE2, D) of the query tile in stage S: BS pairs, filled by a DMA of its own
// alongside the tile's, so a step reads them from LDS.  1 KiB: one DMA
// instruction (64 lanes x 16 bytes); at block 64 its upper half holds a copy.
template <int BS, int S>
struct RowStats {
  static __device__ __forceinline__ char* buf() {
    __shared__ __attribute__((aligned(1024))) char b[1024];
    return b;
  }
};

// One 64 x 16-byte DMA into LDS at the wave-uniform address m0v (+16 per
// lane) from base + off (per lane).  The leading s_nop 4 gives the 5 wait
// states an SGPR written by a vector instruction needs before a vector-memory
// instruction reads it; the M0 write gets its 1.
__device__ __forceinline__ void dma16x1(gchar_ptr base, uint32_t off, uint32_t m0v) {
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(m0v)
               : "memory", "m0");
}

// Wave 0 fetches the (LSE2, D) pairs of query tile `tile` into stage S: lane
// l takes pairs 2 (l mod BS/2) .. +1 (16 bytes; the rows of one (b, h) stay
// inside it).
template <int BS, int S>
__device__ __forceinline__ void issue_rowstats(gchar_ptr rs_bh, int tile, int wave, int lane) {
  if (wave != 0) return;
  const uint32_t off = static_cast<uint32_t>((tile * BS + 2 * (lane % (BS / 2))) * 8);
  dma16x1(rs_bh, off, __builtin_amdgcn_readfirstlane(lds_addr(RowStats<BS, S>::buf())));
}

// One query tile: this wave's 32 keys x its 32 queries of the tile.
template <typename T, int BS, int S, bool QM>
__device__ __forceinline__ void step_kv(KvState& st, const u32x4 (&kop)[Cfg<T, BS>::QC],
                                        const u32x4 (&vop)[Cfg<T, BS>::QC], float kbias_c, bool last,
                                        int tile_u, int tile_fill, gchar_ptr qbh, gchar_ptr gbh,
                                        gchar_ptr rs_bh, int wave, int lane, int wq, const uint8_t* qpad_b) {
  const int qb = wq * 32, g = lane >> 5;
  // Pair masking with padded keys in this unit: the pad bytes of this wave's
  // 32 query rows of the tile (null otherwise), loaded before the wait.
  PadWords qw;
  if constexpr (QM) {
    if (qpad_b != nullptr) {
      qw = load_pad(qpad_b + static_cast<size_t>(tile_u) * BS, qb);
      asm volatile("" ::: "memory");
    }
  }
  __builtin_amdgcn_s_waitcnt(7 << 4);
  ring_barrier();
  // (LSE2, D) of this lane's 16 accumulator rows (two runs of 8 queries), from LDS
  const char* rsl = RowStats<BS, S>::buf() + (qb + 8 * g) * 8;
  f32x4 l4[4], d4[4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(rsl + (16 * h + 4 * x) * 8);
      const f32x4 c = *reinterpret_cast<const f32x4*>(rsl + (16 * h + 4 * x) * 8 + 16);
      l4[2 * h + x] = {a[0], a[2], c[0], c[2]};
      d4[2 * h + x] = {a[1], a[3], c[1], c[3]};
    }
  const f32x16 s = rows_times<T, BS, S, 0>(kop, qb, lane);    // S = Q K^T (rows = queries)
  const f32x16 dp = rows_times<T, BS, S, 1>(vop, qb, lane);   // dP = dO V^T
  const VOp<T> got = cols_op<T, BS, S, 1>(qb, lane);         // dO^T
  const VOp<T> qt = cols_op<T, BS, S, 0>(qb, lane);          // Q^T
  // Pair masking: bit i of rpad set when query qb + i of the tile is padding;
  // such a row takes no key offsets (its uniform offset cancels).
  uint32_t rpad = 0;
  if constexpr (QM) {
    if (qpad_b != nullptr)
      rpad = zero_byte_mask(qw.p[0]) | (zero_byte_mask(qw.p[1]) << 8) | (zero_byte_mask(qw.p[2]) << 16) |
             (zero_byte_mask(qw.p[3]) << 24);
  }
  float p[16], ds[16];
  if (rpad == 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float l2 = l4[v >> 2][v & 3], dd = d4[v >> 2][v & 3];
      p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], kScaleLog2, kbias_c - l2));
      ds[v] = p[v] * (dp[v] - dd);
    }
  } else {
    // element v of this lane is query qb + 16 (v / 8) + 8 g + 4 ((v / 4) % 2) + v % 4
    const uint32_t rg = rpad >> (8 * g);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float l2 = l4[v >> 2][v & 3], dd = d4[v >> 2][v & 3];
      const float kb = (rg >> (16 * (v >> 3) + 4 * ((v >> 2) & 1) + (v & 3))) & 1u ? 0.0f : kbias_c;
      p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], kScaleLog2, kb - l2));
      ds[v] = p[v] * (dp[v] - dd);
    }
  }
  if constexpr (sizeof(T) == 2) {
    bf16x8 pb[2], db[2];
    pack_pairs(p, pb);
    pack_pairs(ds, db);
    if (!last) {
      issue_tile<T, BS, S ^ 1>(qbh, gbh, tile_fill, wave, lane);
      issue_rowstats<BS, S ^ 1>(rs_bh, tile_fill, wave, lane);
    }
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
        st.dv[dh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(got.a[dh][mm], pb[mm], st.dv[dh], 0, 0, 0);
        st.dk[dh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt.a[dh][mm], db[mm], st.dk[dh], 0, 0, 0);
      }
  } else {
    if (!last) {
      issue_tile<T, BS, S ^ 1>(qbh, gbh, tile_fill, wave, lane);
      issue_rowstats<BS, S ^ 1>(rs_bh, tile_fill, wave, lane);
    }
    tprod(st.dv, got, p);
    tprod(st.dk, qt, ds);
  }
}

// Sum of the two query groups' dK^T and dV^T (wave wq keeps dims
// [32 wq, 32 wq + 32)), exchanged through both stages; dK scaled by 1/sqrt(d).
template <typename T, int BS, int KEEP>
__device__ __forceinline__ void finalize_kv_half(KvState& st, const KvUnit& w, int wk, int lane) {
  using C = Cfg<T, BS>;
  constexpr int GIVE = KEEP ^ 1;
  float* xv = reinterpret_cast<float*>(Stage<T, BS, 0>::k());   // 16 KB: dV halves
  float* xk = reinterpret_cast<float*>(Stage<T, BS, 1>::k());   // 16 KB: dK halves
  const int mine = (wk * 2 + KEEP) * 16, theirs = (wk * 2 + GIVE) * 16;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    xv[(mine + v) * 64 + lane] = st.dv[GIVE][v];
    xk[(mine + v) * 64 + lane] = st.dk[GIVE][v];
  }
  lds_barrier();
  const int j = lane & 31, g = lane >> 5;
  float yv[2][8], yk[2][8];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      yv[h8][e] = st.dv[KEEP][8 * h8 + e] + xv[(theirs + 8 * h8 + e) * 64 + lane];
      yk[h8][e] = (st.dk[KEEP][8 * h8 + e] + xk[(theirs + 8 * h8 + e) * 64 + lane]);
    }
  const bargs_ptr b = bargs();
  if (w.gsel < 0) {
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
      for (int e = 0; e < 8; ++e) yk[h8][e] *= 0.125f;   // 1/sqrt(64)
    const size_t ro = w.off + static_cast<size_t>(w.k0 + wk * 32 + j) * C::ROWB;
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      store_row8(b->dv + ro + (KEEP * 32 + 16 * h8 + 8 * g) * C::ES, yv[h8], static_cast<T*>(nullptr));
      store_row8(b->dk + ro + (KEEP * 32 + 16 * h8 + 8 * g) * C::ES, yk[h8], static_cast<T*>(nullptr));
    }
    return;
  }
  float* bv = b->dv_part + w.pbase * kD;
  float* bk = b->dk_part + w.pbase * kD;
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 v4 = {yv[h8][4 * hf], yv[h8][4 * hf + 1], yv[h8][4 * hf + 2], yv[h8][4 * hf + 3]};
      const f32x4 k4 = {yk[h8][4 * hf], yk[h8][4 * hf + 1], yk[h8][4 * hf + 2], yk[h8][4 * hf + 3]};
      *reinterpret_cast<f32x4*>(bv + partial_slot(wk, KEEP, 2 * h8 + hf, lane)) = v4;
      *reinterpret_cast<f32x4*>(bk + partial_slot(wk, KEEP, 2 * h8 + hf, lane)) = k4;
    }
}

// End of a dK/dV unit: the query groups' dK^T and dV^T summed -- for four
// query groups (block 128) first 2,3 -> 0,1 in full (dV through stage 0, dK
// through stage 1), then 0 <-> 1 by head dims.
template <typename T, int BS>
__device__ __forceinline__ void finalize_kv(KvState& st, const KvUnit& w, int wq, int wk, int lane) {
  lds_barrier();   // every wave is past its last LDS read of the unit
  if constexpr (BS / 32 == 4) {
    float* xv = reinterpret_cast<float*>(Stage<T, BS, 0>::k());
    float* xk = reinterpret_cast<float*>(Stage<T, BS, 1>::k());
    if (wq >= 2) {
      const int slot = ((wq - 2) * 2 + wk) * 32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        xv[(slot + v) * 64 + lane] = st.dv[0][v];
        xv[(slot + 16 + v) * 64 + lane] = st.dv[1][v];
        xk[(slot + v) * 64 + lane] = st.dk[0][v];
        xk[(slot + 16 + v) * 64 + lane] = st.dk[1][v];
      }
    }
    lds_barrier();
    if (wq < 2) {
      const int slot = (wq * 2 + wk) * 32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        st.dv[0][v] += xv[(slot + v) * 64 + lane];
        st.dv[1][v] += xv[(slot + 16 + v) * 64 + lane];
        st.dk[0][v] += xk[(slot + v) * 64 + lane];
        st.dk[1][v] += xk[(slot + 16 + v) * 64 + lane];
      }
    }
    lds_barrier();
  }
  if (wq == 0)
    finalize_kv_half<T, BS, 0>(st, w, wk, lane);
  else if (wq == 1)
    finalize_kv_half<T, BS, 1>(st, w, wk, lane);
  else
    lds_barrier();   // query groups 2 and 3: the last round's barrier
}

template <typename T, int BS, bool HAS_PAD, bool QM, int KIND>
__device__ __forceinline__ void run_dkdv(int n_units) {
  using C = Cfg<T, BS>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // two key groups (32 keys each) of the 64-key unit, BS/32 query groups of each query tile
  const int wk = wave & 1, wq = wave >> 1;
  int first, stride, end;
  {
    const int G = gridDim.x, x = blockIdx.x;
    if ((G & 7) == 0) {
      const int X = x & 7;
      first = static_cast<int>((static_cast<long long>(n_units) * X) >> 3) + (x >> 3);
      end = static_cast<int>((static_cast<long long>(n_units) * (X + 1)) >> 3);
      stride = G >> 3;
    } else {
      first = x;
      end = n_units;
      stride = G;
    }
  }
  if (first >= end) return;
  Cursor cur = cursor_at<T, BS, KIND>(kargs(), first);
  for (;;) {
    const bargs_ptr b = bargs();
    const KvUnit cu = decode_kv_unit<T, BS, KIND>(b, cur);
    // K^T and V^T of this wave's 32 keys as B operands (lane j: key k0 + 32 wk + j)
    u32x4 kop[C::QC], vop[C::QC];
    load_q<T, BS>(b->f.k + cu.off + static_cast<size_t>(cu.k0) * C::ROWB, wk, lane, kop);
    load_q<T, BS>(b->f.v + cu.off + static_cast<size_t>(cu.k0) * C::ROWB, wk, lane, vop);
    float kbias_c = 0.0f;
    const uint8_t* qpad_b = nullptr;   // query pad bytes, when pair masking has key offsets to take back
    if constexpr (HAS_PAD) {
      const uint8_t pv = b->f.pad[static_cast<size_t>(cu.b) * b->f.L + cu.k0 + wk * 32 + (lane & 31)];
      kbias_c = pv == 0 ? kMaskRaw * kScaleLog2 : 0.0f;
      if constexpr (QM) {
        if (__any(pv == 0)) qpad_b = b->f.pad + static_cast<size_t>(cu.b) * b->f.L;
      }
    }
    const gchar_ptr qbh = (gchar_ptr)(b->f.q) + cu.off, gbh = (gchar_ptr)(b->dout) + cu.off;
    const gchar_ptr rs_bh = (gchar_ptr)(b->rowstat + static_cast<size_t>(cu.bh) * b->f.L);
    issue_tile<T, BS, 0>(qbh, gbh, kv_tile_at(cu.tl, 0), wave, lane);
    issue_rowstats<BS, 0>(rs_bh, kv_tile_at(cu.tl, 0), wave, lane);
    KvState st;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      st.dk[0][v] = 0.0f;
      st.dk[1][v] = 0.0f;
      st.dv[0][v] = 0.0f;
      st.dv[1][v] = 0.0f;
    }
    const int ntiles = cu.ntiles;
    constexpr int TRIP = 12;
    for (int u = 0; u < ntiles; u += TRIP) {
      int rem = ntiles - u;
      asm volatile("" : "+s"(rem));
      uint32_t tp[(TRIP + 2) / 2];
#pragma unroll
      for (int k = 0; k < (TRIP + 2) / 2; ++k) {
        const uint32_t t0 = 2 * k < rem ? static_cast<uint32_t>(kv_tile_at(cu.tl, u + 2 * k)) : 0u;
        const uint32_t t1 = 2 * k + 1 < rem ? static_cast<uint32_t>(kv_tile_at(cu.tl, u + 2 * k + 1)) : 0u;
        tp[k] = t0 | (t1 << 16);
      }
#define BB_TILE(k) static_cast<int>((tp[(k) >> 1] >> (16 * ((k) & 1))) & 0xffffu)
#define BB_STEP(k)                                                                                    \
  if ((k) < rem)                                                                                      \
    step_kv<T, BS, (k) % 2, QM>(st, kop, vop, kbias_c, (k) + 1 == rem, BB_TILE(k), BB_TILE((k) + 1), qbh, \
                            gbh, rs_bh, wave, lane, wq, qpad_b);
      BB_STEP(0) BB_STEP(1) BB_STEP(2) BB_STEP(3) BB_STEP(4) BB_STEP(5)
      BB_STEP(6) BB_STEP(7) BB_STEP(8) BB_STEP(9) BB_STEP(10) BB_STEP(11)
#undef BB_STEP
#undef BB_TILE
    }
    finalize_kv<T, BS>(st, cu, wq, wk, lane);
    lds_barrier();
    cur = cursor_advance<T, BS, KIND>(kargs(), cur, stride);
    if (cur.unit >= end) break;
  }
}

// Sums of the split-K partials: KIND 0, dQ rows of query blocks 0 and nb-1,
// dK and dV rows of key blocks 0 and nb-1; KIND 3, the rows of every block of
// the three.  Workgroup: 8 rows x 64 dims of one 32-row group of one block of
// one matrix; thread (q, g, jj) as in the forward's merge; chunks summed in
// order.
template <typename T, int BS, int KIND>
__global__ void __launch_bounds__(64) bb_bwd_reduce_kernel(BwdArgs a) {
  constexpr int ROWB = kD * sizeof(T);
  constexpr int UB = BS / 64;                                 // 64-row blocks per block
  const int rb = blockIdx.x & 3;
  const int grp = (blockIdx.x >> 2) & 1;
  int rest = blockIdx.x >> 3;
  const int ub = rest % UB;
  rest /= UB;
  const int mat = rest % 3, gblk = rest / 3;
  int bh, blkid, nsum;
  size_t base;
  if constexpr (KIND == 3) {
    const int nb = a.f.nb, gc = a.f.gc, mc = a.f.mc;
    bh = gblk / nb;
    blkid = gblk - bh * nb;
    const int slot0 = blkid == 0 ? 0 : (blkid == nb - 1 ? gc : 2 * gc + (blkid - 1) * mc);
    nsum = blkid == 0 || blkid == nb - 1 ? gc : mc;
    base = static_cast<size_t>(bh) * (2 * gc + (nb - 2) * mc) + slot0;
  } else {
    bh = gblk >> 1;
    const int gsel = gblk & 1;
    blkid = gsel ? a.f.nb - 1 : 0;
    nsum = a.f.n_s;
    base = (static_cast<size_t>(bh) * 2 + gsel) * a.f.n_s;
  }
  const int t = threadIdx.x;
  const int q = t >> 4, g = (t >> 3) & 1, j = rb * 8 + (t & 7);
  const int lane = j + 32 * g;
  const int row = ub * 64 + grp * 32 + j;
  const float* part = mat == 0 ? a.dq_part : (mat == 1 ? a.dk_part : a.dv_part);
  char* dst = mat == 0 ? a.dq : (mat == 1 ? a.dk : a.dv);
  f32x4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  // four chunks' loads in flight before their adds (the adds stay in chunk
  // order); one at a time, each chunk waited out the previous one's latency
  const float* p0 = part + (base * BS + ub * 64) * kD;
  constexpr size_t CH = static_cast<size_t>(BS) * kD;        // floats per chunk
  const int o0 = partial_slot(grp, 0, q, lane), o1 = partial_slot(grp, 1, q, lane);
  int s = 0;
  for (; s + 4 <= nsum; s += 4) {
    f32x4 x[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i][0] = *reinterpret_cast<const f32x4*>(p0 + (s + i) * CH + o0);
      x[i][1] = *reinterpret_cast<const f32x4*>(p0 + (s + i) * CH + o1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[0] += x[i][0];
      acc[1] += x[i][1];
    }
  }
  for (; s < nsum; ++s) {
    acc[0] += *reinterpret_cast<const f32x4*>(p0 + s * CH + o0);
    acc[1] += *reinterpret_cast<const f32x4*>(p0 + s * CH + o1);
  }
  const float sc = mat == 2 ? 1.0f : 0.125f;   // dQ and dK carry 1/sqrt(64)
  char* orow = dst + (static_cast<size_t>(bh) * a.f.L + static_cast<size_t>(blkid) * BS + row) * ROWB;
#pragma unroll
  for (int keep = 0; keep < 2; ++keep) {
    const int d0 = 32 * keep + 16 * (q >> 1) + 8 * g + 4 * (q & 1);
    store_f32x4(orow + d0 * sizeof(T), acc[keep] * sc, static_cast<T*>(nullptr));
  }
}

// (bf16, block 64: a register budget of 2 waves per SIMD; the kernel then
// allocates 168 registers without spilling, which still gives 3 waves per
// SIMD -- a budget of 3 made the compiler fit 168 with 4 spills at the unit
// boundaries, 1.6% slower.  Block 128 keeps the budget of 3: with 2 its padded
// form grows to 221 registers, 2 waves per SIMD.)
// QM: pair masking (BB_QUERY_MASK), its own instantiation so that the usual
// kernels keep their registers.
// KIND: 0 ordinary units, 3 the small-problem split.
template <typename T, int BS, bool HAS_PAD, bool QM, int KIND>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? (BS == 64 ? 2 : 3) : (BS == 64 ? 1 : 2)))) bb_bwd_dq_kernel(BwdArgs, int n_units) {
  run_dq<T, BS, HAS_PAD, QM, KIND>(n_units);
}
template <typename T, int BS, bool HAS_PAD, bool QM, int KIND>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : (BS == 64 ? 1 : 2)))) bb_bwd_dkdv_kernel(BwdArgs, int n_units) {
  run_dkdv<T, BS, HAS_PAD, QM, KIND>(n_units);
}


// ================================================================== layer ==
// Projections of the attention layer (the page's layer construction: input
// projections of the hidden states to query, key and value, key_dim =
// hidden / heads, and an output projection of the concatenated heads):
//   C = A W^T + bias, bf16 operands, fp32 accumulation, bf16 results.
//   A: MODE 0 the hidden states x [M = B*L][K = hidden];
//      MODE 1 the attention output in its head-split layout [B][H][L][64]
//      (k = 64 h + dd: one K step of 64 is one head, 128 contiguous rows).
//   W: [N][K], the [out][in] layout of a linear layer.
//   C: MODE 0 q, k and v in the attention's layout [B][H][L][64] (columns
//      n of [q | k | v], N = 3*hidden); MODE 1 y [M][N].
// Workgroup tile 32 SMW WMW rows of A x 64 SN rows of W, with 2 WMW waves of
// 32 SMW x 32 SN (SMW x SN subtiles of 32 x 32 each); K in steps of 64 through a
// two-stage LDS ring filled by the same DMA as the attention.  Computed
// transposed (C^T = W A^T): lane = row of A, 16 accumulators = 2 runs of 8
// consecutive columns, so the epilogue writes 16-byte runs with the bias
// added.

struct ProjArgs {
  const char* a;
  const char* w;
  const float* bias;
  char* out;
  int M, N, K;
  int L, H;      // sequence length, heads (head-split layouts)
  int hidden;
};

// Two DMAs of 64 x 16 bytes from one wave-uniform base (see dma16x4).
__device__ __forceinline__ void dma16x2(gchar_ptr base, uint32_t o0, uint32_t o1, uint32_t m0a, uint32_t m0b) {
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %4\n\t"
      "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %4"
      :
      : "v"(o0), "v"(o1), "s"(m0a), "s"(m0b), "s"(base)
      : "memory", "m0");
}

// Tile order of the projections.  Consecutive workgroups go round-robin to
// the 8 XCDs, each with its own L2: when the row panels split evenly, XCD x
// takes panels [x pm, (x+1) pm) and walks them in groups of GM panels, column
// tile by column tile, so the A panels and W tiles its resident workgroups
// share stay in its L2 (one read of the layer's A per XCD instead of per tile
// column).
__device__ __forceinline__ void proj_tile(int tiles_m, int tiles_n, int& tm, int& tn) {
  if ((tiles_m & 7) == 0) {
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int pm = tiles_m >> 3;
    const int GM = pm % 8 == 0 ? 8 : (pm % 4 == 0 ? 4 : 1);
    const int grp = idx / (GM * tiles_n), rr = idx - grp * (GM * tiles_n);
    tm = xcd * pm + grp * GM + rr % GM;
    tn = rr / GM;
  } else {
    tm = blockIdx.x / tiles_n;
    tn = blockIdx.x - tm * tiles_n;
  }
}

// Epilogue of a wave's SN x SMW subtiles of C^T: lane (j, gh) holds C[m][n]
// for m = mw + 32 ms + j and n = nw + 32 ns + 16 h + 8 gh + (0..7); the bias
// is added and each run of 8 columns is one 16-byte store.
template <int MODE, int SMW, int SN>
__device__ __forceinline__ void proj_epilogue(const ProjArgs& g, const f32x16 (&acc)[SN][SMW], int mw, int nw,
                                              int j, int gh) {
#pragma unroll
  for (int ns = 0; ns < SN; ++ns)
#pragma unroll
    for (int ms = 0; ms < SMW; ++ms) {
      const int m = mw + ms * 32 + j;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = nw + ns * 32 + 16 * h + 8 * gh;
        const f32x4 b0v = *reinterpret_cast<const f32x4*>(g.bias + n);
        const f32x4 b1v = *reinterpret_cast<const f32x4*>(g.bias + n + 4);
        float x8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x8[e] = acc[ns][ms][8 * h + e] + b0v[e];
          x8[4 + e] = acc[ns][ms][8 * h + 4 + e] + b1v[e];
        }
        char* dst;
        if (MODE == 0) {
          const int which = n / g.hidden, nn = n - which * g.hidden;
          const int hh = nn >> 6, dd = nn & 63;
          const int bb = m / g.L, l = m - bb * g.L;
          dst = g.out + static_cast<size_t>(which) * g.M * g.hidden * 2 +
                ((static_cast<size_t>(bb) * g.H + hh) * g.L + l) * 128 + dd * 2;
        } else {
          dst = g.out + (static_cast<size_t>(m) * g.N + n) * 2;
        }
        store_row8(dst, x8, static_cast<__bf16*>(nullptr));
      }
    }
}

template <int MODE, int WMW, int SMW, int SN>
__global__ void __launch_bounds__(128 * WMW) __attribute__((amdgpu_waves_per_eu(SMW > 2 ? 1 : 2)))
bb_proj_kernel(ProjArgs g) {
  constexpr int NW = 2 * WMW;                      // waves: WMW along A rows x 2 along W rows
  constexpr int TM = 32 * SMW * WMW, TN = 64 * SN;  // rows of A and of W per tile
  constexpr int AB = TM * 128, SB = AB + TN * 128;  // bytes per stage (128-byte rows): A part, whole
  constexpr int NA = AB / 1024 / NW, NWI = TN * 128 / 1024 / NW;   // DMAs per wave per stage
  static_assert(NA % 2 == 0 && NA * NW * 1024 == AB && NWI * NW * 1024 == TN * 128, "DMAs split evenly");
  __shared__ __attribute__((aligned(1024))) char lds[2 * SB];   // [stage][A rows | W rows]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WMW, wn = wave / WMW;
  const int j = lane & 31, gh = lane >> 5;
  const int tiles_n = g.N / TN;
  const int tiles_m = g.M / TM;
  int tm, tn;
  proj_tile(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * TM, n0 = tn * TN;
  const int nk = g.K / 64;
  // A rows of this tile: MODE 1 reads head ks of batch b, rows l0 .. l0+TM-1
  const int b0 = m0 / g.L, l0 = m0 - b0 * g.L;
  const size_t a_row = MODE == 0 ? static_cast<size_t>(g.K) * 2 : 128;
  // This wave's DMA instructions per stage: A instructions wave + NW jj, W
  // instructions wave + NW jj.  Lane l of instruction i fills physical chunk
  // slot 64 i + l: row (64 i + l) / 8, chunk l % 8, with the logical chunk
  // the swizzle puts there (A: row & 7, W: swz_k, as the operand reads below).
  uint32_t ao[NA], wo[NWI], am[NA], wmo[NWI];
  const uint32_t lds0 = lds_addr(lds);
#pragma unroll
  for (int jj = 0; jj < NA; ++jj) {
    const int ins = wave + NW * jj;
    const int row = (ins * 64 + lane) >> 3, p = lane & 7;
    ao[jj] = static_cast<uint32_t>(row * a_row + ((p ^ (row & 7)) << 4));
    am[jj] = ins * 1024;
  }
#pragma unroll
  for (int jj = 0; jj < NWI; ++jj) {
    const int ins = wave + NW * jj;
    const int row = (ins * 64 + lane) >> 3, p = lane & 7;
    wo[jj] = static_cast<uint32_t>(static_cast<size_t>(row) * g.K * 2 + ((p ^ swz_k(row)) << 4));
    wmo[jj] = AB + ins * 1024;
  }
  auto issue = [&](int ks, int st) {
    const gchar_ptr ab = MODE == 0
        ? (gchar_ptr)(g.a) + static_cast<size_t>(m0) * g.K * 2 + static_cast<size_t>(ks) * 128
        : (gchar_ptr)(g.a) + ((static_cast<size_t>(b0) * g.H + ks) * g.L + l0) * 128;
    const gchar_ptr wb = (gchar_ptr)(g.w) + static_cast<size_t>(n0) * g.K * 2 + static_cast<size_t>(ks) * 128;
    const uint32_t base = lds0 + st * SB;
#pragma unroll
    for (int jj = 0; jj < NA; jj += 2)
      dma16x2(ab, ao[jj], ao[jj + 1], __builtin_amdgcn_readfirstlane(base + am[jj]),
              __builtin_amdgcn_readfirstlane(base + am[jj + 1]));
#pragma unroll
    for (int jj = 0; jj + 1 < NWI; jj += 2)
      dma16x2(wb, wo[jj], wo[jj + 1], __builtin_amdgcn_readfirstlane(base + wmo[jj]),
              __builtin_amdgcn_readfirstlane(base + wmo[jj + 1]));
    if constexpr (NWI % 2 == 1)
      dma16x1(wb, wo[NWI - 1], __builtin_amdgcn_readfirstlane(base + wmo[NWI - 1]));
  };
  f32x16 acc[SN][SMW];
#pragma unroll
  for (int x = 0; x < SN; ++x)
#pragma unroll
    for (int y = 0; y < SMW; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
  issue(0, 0);
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks & 1;
    __builtin_amdgcn_s_waitcnt(7 << 4);
    ring_barrier();
    if (ks + 1 < nk) issue(ks + 1, st ^ 1);
    const char* la = lds + st * SB;
    const char* lw = la + AB;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      u32x4 bop[SMW], aop[SN];
#pragma unroll
      for (int ms = 0; ms < SMW; ++ms) {
        const int row = wm * (32 * SMW) + ms * 32 + j;
        bop[ms] = *reinterpret_cast<const u32x4*>(la + row * 128 + (((2 * x + gh) ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int ns = 0; ns < SN; ++ns) {
        const int row = wn * (32 * SN) + ns * 32 + perm_row(j);
        aop[ns] = *reinterpret_cast<const u32x4*>(lw + row * 128 + (((2 * x + gh) ^ swz_k(row)) << 4));
      }
#pragma unroll
      for (int ns = 0; ns < SN; ++ns)
#pragma unroll
        for (int ms = 0; ms < SMW; ++ms)
          acc[ns][ms] = mfma_qk(aop[ns], bop[ms], acc[ns][ms], static_cast<__bf16*>(nullptr));
    }
  }
  proj_epilogue<MODE, SMW, SN>(g, acc, m0 + wm * (32 * SMW), n0 + wn * (32 * SN), j, gh);
}

// Launch C = A W^T + bias for one projection: tiles of 128 rows of A by 192
// rows of W where N allows (3 hidden always does), else 128.
template <int MODE>
void launch_proj(const ProjArgs& a, hipStream_t s) {
  if (a.N % 192 == 0)
    hipLaunchKernelGGL((bb_proj_kernel<MODE, 2, 2, 3>), dim3(static_cast<unsigned>((a.M / 128) * (a.N / 192))),
                       dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bb_proj_kernel<MODE, 2, 2, 2>), dim3(static_cast<unsigned>((a.M / 128) * (a.N / 128))),
                       dim3(256), 0, s, a);
}

// ---------------------------------------------------------------- host side --

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
  size_t pm, pl, po, total;
};

// Problems whose ordinary units (one per 64 query rows of a query block, the
// global blocks split into kChunkTiles-tile chunks) number fewer than
// kSmallUnits leave most of the chip idle and take one unit's latency.  They
// run kind 3 units instead: every query block split over its key tiles into
// the fewest chunks for which the units still number at most kSmallSlots /
// (block / 64), one workgroup per compute unit (two workgroups sharing a
// compute unit's matrix cores measured slower than one unit of twice the
// tiles).  The choice depends on the sizes only, so the workspace size can
// bound it.
constexpr long long kSmallUnits = 512;
constexpr long long kSmallSlots = 256;

struct SmallSplit {
  int gc, mc;   // chunks per global / middle query block; 0: ordinary units
};

SmallSplit small_split(int B, int H, int nb, int block, int r) {
  const long long qs = block / 64, bh = static_cast<long long>(B) * H;
  const int n_s = (nb + kChunkTiles - 1) / kChunkTiles;
  const long long normal = bh * (2LL * n_s + nb - 2) * qs;
  if (normal >= kSmallUnits || normal == 0) return {0, 0};
  const int nt_min = 2 + (nb - 2 < 2 ? nb - 2 : 2) + r;   // tiles of blocks 1 and nb-2
  const int nt_max = 2 + (nb - 2 < 3 ? nb - 2 : 3) + r;
  for (int cs = 1; cs <= nb; ++cs) {
    const int gc = (nb + cs - 1) / cs;
    int mc = (nt_max + cs - 1) / cs;
    if (mc > nt_min) mc = nt_min;                            // no chunk may be empty
    const long long units = bh * (2LL * gc + static_cast<long long>(nb - 2) * mc) * qs;
    if (units <= kSmallSlots / qs) return units > normal ? SmallSplit{gc, mc} : SmallSplit{0, 0};
  }
  return {0, 0};
}

Layout workspace_layout(int B, int H, int nb, int block) {
  // partial blocks (block rows each): the global chunks of the ordinary
  // units, or the chunks of every query block for the small-problem split
  // (the largest over every r the sizes allow)
  const size_t bh = static_cast<size_t>(B) * H;
  const size_t n_s = static_cast<size_t>((nb + kChunkTiles - 1) / kChunkTiles);
  size_t blocks = bh * 2 * n_s;
  // (the split needs fewer than kSmallUnits ordinary units, whatever r is)
  const bool can_split = bh * (2 * n_s + nb - 2) * static_cast<size_t>(block / 64) < static_cast<size_t>(kSmallUnits);
  const int r_max = can_split && nb - 5 > 0 ? nb - 5 : 0;
  for (int r = 0; r <= r_max; ++r) {
    const SmallSplit sp = small_split(B, H, nb, block, r);
    const size_t n = bh * (2 * static_cast<size_t>(sp.gc) + static_cast<size_t>(nb - 2) * sp.mc);
    if (sp.gc > 0 && n > blocks) blocks = n;
  }
  Layout w;
  w.pm = 0;
  w.pl = w.pm + align256(blocks * block * sizeof(float));
  w.po = w.pl + align256(blocks * block * sizeof(float));
  w.total = w.po + blocks * block * kD * sizeof(float);
  return w;
}

int check_shape(int B, int H, int L, int d, int block, int r, int* nb_out) {
  if (B < 0 || H < 0 || L <= 0 || r < 0) return BB_ERR_SHAPE;
  if (d != kD) return BB_ERR_SHAPE;
  if (block != 64 && block != 128) return BB_ERR_SHAPE;
  if (L % block != 0) return BB_ERR_SHAPE;
  const int nb = L / block;
  if (nb < 3 || L / 64 > 65535) return BB_ERR_SHAPE;   // 64-key tile ids fit in 16 bits
  const int r_max = nb - 5 > 0 ? nb - 5 : 0;
  if (r > r_max) return BB_ERR_SHAPE;
  const int n_s = (nb + kChunkTiles - 1) / kChunkTiles;
  const long long units = static_cast<long long>(B) * H * (2LL * n_s + nb - 2) * (block / 64);
  if (units > 0x7fffffffLL) return BB_ERR_SHAPE;
  *nb_out = nb;
  return BB_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

// [a, a + na) and [b, b + nb) share a byte
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Persistent grid for a kernel: as many workgroups as the current device
// holds at once, at most one per unit.  When the device holds fewer than the
// units, rounded down to a multiple of 8 (the XCD count) so that every XCD
// runs the same number; otherwise one workgroup per unit.
int persistent_grid(const void* kernel, int nt, long long n_units, unsigned* grid) {
  int dev = 0, ncu = 0, occ = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BB_ERR_HIP;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return BB_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, nt, 0) != hipSuccess) return BB_ERR_HIP;
  long long g = static_cast<long long>(ncu > 0 ? ncu : 1) * (occ > 0 ? occ : 1);
  if (g >= n_units)
    g = n_units;
  else if (g >= 8)
    g -= g % 8;
  *grid = static_cast<unsigned>(g);
  return BB_OK;
}

// Kernel launches of one call.  `ev0` / `ev1` (may be null): timestamps of
// the start of the first and the end of the last kernel launched here (taken
// by the launches themselves, hipExtLaunchKernelGGL, so they bracket the
// kernels exactly).
template <typename T, int BS, bool HAS_PAD>
int launch(const Args& a, int B, int H, hipStream_t stream, unsigned flags, hipEvent_t ev0, hipEvent_t ev1) {
  using C = Cfg<T, BS>;
  const long long bhs = static_cast<long long>(B) * H;
  const long long per_g = 2LL * a.n_s * C::QSPLIT, per_m = static_cast<long long>(a.nb - 2) * C::QSPLIT;
  const bool units = !(flags & BB_PHASE_MERGE) || (flags & BB_PHASE_UNITS);
  const bool merge = !(flags & BB_PHASE_UNITS) || (flags & BB_PHASE_MERGE);
  unsigned grid = 0;
  int st = BB_OK;
  // bf16 at block 128: the 32-key-step kernels (2 waves of complete rows);
  // otherwise the key-group kernels of run() (32 x 32 subtiles per wave)
  typedef void (*UnitKernel)(Args, int);
  UnitKernel k_fused, k_global, k_middle;
  int nt;
  if constexpr (sizeof(T) == 2 && BS == 128) {
    k_fused = bb_sub32_fused_kernel<BS, HAS_PAD>;
    k_global = bb_sub32_global_rows_kernel<BS, HAS_PAD>;
    k_middle = bb_sub32_middle_rows_kernel<BS, HAS_PAD>;
    nt = kSub32NT;
  } else {
    k_fused = bb_fused_kernel<T, BS, HAS_PAD>;
    k_global = bb_global_rows_kernel<T, BS, HAS_PAD>;
    k_middle = bb_middle_rows_kernel<T, BS, HAS_PAD>;
    nt = C::NT;
  }
  // small problems (a.gc > 0, key-group kernels only): one launch of kind 3
  // units, every query block merged after it
  bool small = false;
  if constexpr (!(sizeof(T) == 2 && BS == 128)) {
    small = a.gc > 0;
    if (units && small) {
      hipEvent_t e1 = merge ? nullptr : ev1;
      const long long n = bhs * (2LL * a.gc + static_cast<long long>(a.nb - 2) * a.mc) * C::QSPLIT;
      st = persistent_grid(reinterpret_cast<const void*>(bb_small_kernel<T, BS, HAS_PAD>), nt, n, &grid);
      if (st != BB_OK) return st;
      hipExtLaunchKernelGGL(bb_small_kernel<T, BS, HAS_PAD>, dim3(grid), dim3(nt), 0, stream, ev0, e1, 0, a,
                            static_cast<int>(n));
      if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
    }
  }
  if (units && !small) {
    hipEvent_t e1 = merge ? nullptr : ev1;
    if (flags & BB_LAUNCH_SPLIT) {
      st = persistent_grid(reinterpret_cast<const void*>(k_global), nt, bhs * per_g, &grid);
      if (st != BB_OK) return st;
      hipExtLaunchKernelGGL(k_global, dim3(grid), dim3(nt), 0, stream, ev0, nullptr, 0, a,
                            static_cast<int>(bhs * per_g));
      if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
      st = persistent_grid(reinterpret_cast<const void*>(k_middle), nt, bhs * per_m, &grid);
      if (st != BB_OK) return st;
      hipExtLaunchKernelGGL(k_middle, dim3(grid), dim3(nt), 0, stream, nullptr, e1, 0, a,
                            static_cast<int>(bhs * per_m));
    } else {
      st = persistent_grid(reinterpret_cast<const void*>(k_fused), nt, bhs * (per_g + per_m), &grid);
      if (st != BB_OK) return st;
      hipExtLaunchKernelGGL(k_fused, dim3(grid), dim3(nt), 0, stream, ev0, e1, 0, a,
                            static_cast<int>(bhs * (per_g + per_m)));
    }
    if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
  }
  if (merge) {
    // 8 workgroups per 64 query rows of every merged block
    if constexpr (!(sizeof(T) == 2 && BS == 128)) {
      if (small)
        hipExtLaunchKernelGGL(bb_global_merge_kernel<T, BS, true>,
                              dim3(static_cast<unsigned>(bhs * a.nb) * (BS / 64) * 2 * 4), dim3(64 * kMergeSplit), 0,
                              stream, units ? nullptr : ev0, ev1, 0, a);
    }
    if (!small)
      hipExtLaunchKernelGGL(bb_global_merge_kernel<T, BS, false>,
                            dim3(static_cast<unsigned>(bhs) * 2 * (BS / 64) * 2 * 4), dim3(64 * kMergeSplit), 0,
                            stream, units ? nullptr : ev0, ev1, 0, a);
    if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
  }
  return BB_OK;
}

}  // namespace

extern "C" int bb_abi_version(void) { return BB_ABI_VERSION; }

extern "C" const char* bb_status_str(int status) {
  switch (status) {
    case BB_OK: return "ok";
    case BB_ERR_NULL: return "a required pointer is NULL";
    case BB_ERR_SHAPE: return "unsupported or inconsistent sizes (d must be 64, block 64 or 128, "
                              "L a multiple of block with at least 3 blocks, 0 <= r <= min(16, nb-5))";
    case BB_ERR_DTYPE: return "dtype must be BB_FP32 or BB_BF16";
    case BB_ERR_RAND_IDX: return "random-block table violates its constraints";
    case BB_ERR_WORKSPACE: return "workspace smaller than bb_attn_workspace_bytes()";
    case BB_ERR_HIP: return "HIP kernel launch failed";
    case BB_ERR_ALIAS: return "out overlaps q, k or v";
    case BB_ERR_ALIGN: return "device pointer misaligned (q/k/v/out 16 B, pad_mask 8 B, workspace 256 B)";
    default: return "unknown status";
  }
}

extern "C" int bb_attn_forward_plan(int B, int H, int L, int d, int block, int r, int dtype, unsigned flags,
                                    long long* n_units, int* small) {
  if (!n_units || !small) return BB_ERR_NULL;
  if (dtype != BB_FP32 && dtype != BB_BF16) return BB_ERR_DTYPE;
  if (flags & ~(BB_LAUNCH_SPLIT | BB_PHASE_UNITS | BB_PHASE_MERGE | BB_QUERY_MASK | BB_ORDINARY_UNITS))
    return BB_ERR_SHAPE;
  int nb = 0;
  const int st = check_shape(B, H, L, d, block, r, &nb);
  if (st != BB_OK) return st;
  const long long bh = static_cast<long long>(B) * H, qs = block / 64;
  SmallSplit sp{0, 0};
  if (!(dtype == BB_BF16 && block == 128) && !(flags & BB_ORDINARY_UNITS)) sp = small_split(B, H, nb, block, r);
  const int n_s = (nb + kChunkTiles - 1) / kChunkTiles;
  *n_units = sp.gc > 0 ? bh * (2LL * sp.gc + static_cast<long long>(nb - 2) * sp.mc) * qs
                       : bh * (2LL * n_s + nb - 2) * qs;
  *small = sp.gc > 0 ? 1 : 0;
  return BB_OK;
}

extern "C" size_t bb_attn_workspace_bytes(int B, int H, int L, int d, int block) {
  int nb = 0;
  if (check_shape(B, H, L, d, block, 0, &nb) != BB_OK) return 0;
  if (B == 0 || H == 0) return 0;
  return workspace_layout(B, H, nb, block).total;
}

namespace {

int forward_impl(const void* q, const void* k, const void* v, const uint8_t* pad_mask, const int32_t* rand_idx,
                 int B, int H, int L, int d, int block, int r, void* out, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream, unsigned flags, void* start_event, void* stop_event,
                 float* lse) {
  if (dtype != BB_FP32 && dtype != BB_BF16) return BB_ERR_DTYPE;
  if (flags & ~(BB_LAUNCH_SPLIT | BB_PHASE_UNITS | BB_PHASE_MERGE | BB_QUERY_MASK | BB_ORDINARY_UNITS))
    return BB_ERR_SHAPE;
  int nb = 0;
  const int st = check_shape(B, H, L, d, block, r, &nb);
  if (st != BB_OK) return st;
  if (B == 0 || H == 0) return BB_OK;
  if (!q || !k || !v || !out || !workspace) return BB_ERR_NULL;
  if (r > 0 && !rand_idx) return BB_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return BB_ERR_ALIGN;
  if ((pad_mask && !aligned(pad_mask, 8)) || !aligned(workspace, 256) ||
      (rand_idx && !aligned(rand_idx, 4)))
    return BB_ERR_ALIGN;
  const size_t es = dtype == BB_BF16 ? 2 : 4;
  const size_t bytes = static_cast<size_t>(B) * H * L * d * es;
  if (overlap(out, q, bytes) || overlap(out, k, bytes) || overlap(out, v, bytes)) return BB_ERR_ALIAS;
  const Layout w = workspace_layout(B, H, nb, block);
  if (workspace_bytes < w.total) return BB_ERR_WORKSPACE;

  Args a;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.pad = pad_mask;
  a.rand_idx = rand_idx;
  a.out = static_cast<char*>(out);
  char* ws = static_cast<char*>(workspace);
  a.pm = reinterpret_cast<float*>(ws + w.pm);
  a.pl = reinterpret_cast<float*>(ws + w.pl);
  a.po = reinterpret_cast<float*>(ws + w.po);
  a.lse = lse;
  a.H = H;
  a.L = L;
  a.nb = nb;
  a.r = r;
  a.n_s = (nb + kChunkTiles - 1) / kChunkTiles;
  a.qmask = (flags & BB_QUERY_MASK) && pad_mask != nullptr ? 1 : 0;
  a.gc = a.mc = 0;
  if (!(dtype == BB_BF16 && block == 128) && !(flags & BB_ORDINARY_UNITS)) {   // the key-group kernels
    const SmallSplit sp = small_split(B, H, nb, block, r);
    a.gc = sp.gc;
    a.mc = sp.mc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(start_event), e1 = static_cast<hipEvent_t>(stop_event);
  const bool p = pad_mask != nullptr;
  if (dtype == BB_BF16) {
    if (block == 64)
      return p ? launch<__bf16, 64, true>(a, B, H, s, flags, e0, e1) : launch<__bf16, 64, false>(a, B, H, s, flags, e0, e1);
    return p ? launch<__bf16, 128, true>(a, B, H, s, flags, e0, e1) : launch<__bf16, 128, false>(a, B, H, s, flags, e0, e1);
  }
  if (block == 64)
    return p ? launch<float, 64, true>(a, B, H, s, flags, e0, e1) : launch<float, 64, false>(a, B, H, s, flags, e0, e1);
  return p ? launch<float, 128, true>(a, B, H, s, flags, e0, e1) : launch<float, 128, false>(a, B, H, s, flags, e0, e1);
}

}  // namespace

extern "C" int bb_attn_forward_timed(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                                     const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                                     void* out, int dtype, void* workspace, size_t workspace_bytes,
                                     void* stream, unsigned flags, void* start_event, void* stop_event) {
  return forward_impl(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, dtype, workspace, workspace_bytes,
                      stream, flags, start_event, stop_event, nullptr);
}

extern "C" int bb_attn_forward_lse_ex(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                                      const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                                      void* out, int dtype, void* workspace, size_t workspace_bytes,
                                      void* stream, float* lse, unsigned flags) {
  if (flags & ~(BB_QUERY_MASK | BB_ORDINARY_UNITS)) return BB_ERR_SHAPE;
  if (B > 0 && H > 0 && lse == nullptr) return BB_ERR_NULL;
  if (lse != nullptr && !aligned(lse, 4)) return BB_ERR_ALIGN;
  return forward_impl(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, dtype, workspace, workspace_bytes,
                      stream, BB_LAUNCH_FUSED | flags, nullptr, nullptr, lse);
}

extern "C" int bb_attn_forward_lse(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                                   const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                                   void* out, int dtype, void* workspace, size_t workspace_bytes,
                                   void* stream, float* lse) {
  return bb_attn_forward_lse_ex(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, dtype, workspace,
                                workspace_bytes, stream, lse, 0u);
}

extern "C" int bb_attn_forward_ex(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                                  const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                                  void* out, int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream, unsigned flags) {
  return bb_attn_forward_timed(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, dtype, workspace,
                               workspace_bytes, stream, flags, nullptr, nullptr);
}

extern "C" int bb_attn_forward(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                               const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                               void* out, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return bb_attn_forward_ex(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, dtype, workspace,
                            workspace_bytes, stream, BB_LAUNCH_FUSED);
}


// --------------------------------------------- forward without allocation --
// bb_attn_forward_noalloc keeps the split-K partials in `scratch`, a device
// array of the library's own (each GPU holds its copy from the library's
// load until the process ends).  Host code never passes the array's name to
// a kernel: its device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is kept per device.
static __device__ __align__(256) char scratch[BB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use).
int scratch_of_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BB_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BB_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BB_OK;
}

}  // namespace

extern "C" int bb_attn_forward_noalloc(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                                       const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                                       void* out, int dtype, void* stream) {
  // sizes first (no HIP call on a rejected call), then the scratch address
  int nb = 0;
  if (dtype != BB_FP32 && dtype != BB_BF16) return BB_ERR_DTYPE;
  int st = check_shape(B, H, L, d, block, r, &nb);
  if (st != BB_OK) return st;
  if (B == 0 || H == 0) return BB_OK;
  if (workspace_layout(B, H, nb, block).total > BB_NOALLOC_SCRATCH_BYTES) return BB_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != BB_OK) return st;
  return forward_impl(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, dtype, ws, BB_NOALLOC_SCRATCH_BYTES,
                      stream, BB_LAUNCH_FUSED, nullptr, nullptr, nullptr);
}

// ------------------------------------------------------------ backward host --

namespace {

struct BwdLayout {
  size_t rowstat, dq, dk, dv, total;
};

// The backward's small-problem split (kind 3 units in both passes): with too
// few ordinary units to fill the chip, every query block (dQ) and every key
// block (dK/dV) is split over its tile list into the fewest chunks for which
// the units still number at most kSmallSlots / (block / 64) -- gc chunks per
// global block, mc per middle block, chunks of about the same number of tiles
// (lists of about 8).  mc stays within the shortest middle list of the dK/dV
// pass (its two global rows and band rows), so no chunk is empty; the choice
// does not depend on r, and neither does the workspace.
SmallSplit bwd_split(int B, int H, int nb, int block) {
  const long long qs = block / 64, bh = static_cast<long long>(B) * H;
  const int n_s = (nb + kChunkTiles - 1) / kChunkTiles;
  const long long normal = bh * (2LL * n_s + nb - 2) * qs;
  if (normal >= kSmallUnits || normal == 0) return {0, 0};
  const int mc_max = 2 + (nb - 2 < 2 ? nb - 2 : 2);
  for (int cs = 1; cs <= nb; ++cs) {
    const int gc = (nb + cs - 1) / cs;
    int mc = (8 + cs - 1) / cs;
    if (mc > mc_max) mc = mc_max;
    const long long units = bh * (2LL * gc + static_cast<long long>(nb - 2) * mc) * qs;
    if (units <= kSmallSlots / qs) return units > normal ? SmallSplit{gc, mc} : SmallSplit{0, 0};
  }
  return {0, 0};
}

BwdLayout bwd_layout(int B, int H, int L, int nb, int block) {
  const size_t rows = static_cast<size_t>(B) * H * L;
  const size_t n_s = static_cast<size_t>((nb + kChunkTiles - 1) / kChunkTiles);
  // partial blocks per (b, h): the global blocks' split-K chunks, or the
  // chunks of every block for the small-problem split
  const SmallSplit sp = bwd_split(B, H, nb, block);
  const size_t per_bh = sp.gc > 0 ? 2 * static_cast<size_t>(sp.gc) + static_cast<size_t>(nb - 2) * sp.mc : 0;
  const size_t blocks = per_bh > 2 * n_s ? per_bh : 2 * n_s;
  const size_t part = static_cast<size_t>(B) * H * blocks * block * kD * sizeof(float);
  BwdLayout w;
  w.rowstat = 0;
  w.dq = w.rowstat + align256(rows * 2 * sizeof(float));
  w.dk = w.dq + align256(part);
  w.dv = w.dk + align256(part);
  w.total = w.dv + part;
  return w;
}

template <typename T, int BS, bool HAS_PAD, bool QM, int KIND>
int launch_bwd_kind(const BwdArgs& a, long long n_units, long long reduce_blocks, hipStream_t stream) {
  using C = Cfg<T, BS>;
  unsigned grid = 0;
  int st = persistent_grid(reinterpret_cast<const void*>(&bb_bwd_dq_kernel<T, BS, HAS_PAD, QM, KIND>), C::NT, n_units,
                           &grid);
  if (st != BB_OK) return st;
  hipLaunchKernelGGL((bb_bwd_dq_kernel<T, BS, HAS_PAD, QM, KIND>), dim3(grid), dim3(C::NT), 0, stream, a,
                     static_cast<int>(n_units));
  if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
  st = persistent_grid(reinterpret_cast<const void*>(&bb_bwd_dkdv_kernel<T, BS, HAS_PAD, QM, KIND>), C::NT, n_units,
                       &grid);
  if (st != BB_OK) return st;
  hipLaunchKernelGGL((bb_bwd_dkdv_kernel<T, BS, HAS_PAD, QM, KIND>), dim3(grid), dim3(C::NT), 0, stream, a,
                     static_cast<int>(n_units));
  if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
  // reduce: 8 workgroups per 64 rows of each summed block of each matrix
  hipLaunchKernelGGL((bb_bwd_reduce_kernel<T, BS, KIND>), dim3(static_cast<unsigned>(reduce_blocks * 3 * (BS / 64) * 8)),
                     dim3(64), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
  return BB_OK;
}

template <typename T, int BS, bool HAS_PAD, bool QM>
int launch_bwd(const BwdArgs& a, int B, int H, hipStream_t stream) {
  const long long bhs = static_cast<long long>(B) * H;
  // 64-row query units (dQ) and 64-key units (dK/dV): the same count in either kind
  if (a.f.gc > 0)
    return launch_bwd_kind<T, BS, HAS_PAD, QM, 3>(a, bhs * (2LL * a.f.gc + (a.f.nb - 2LL) * a.f.mc) * (BS / 64),
                                                  bhs * a.f.nb, stream);
  return launch_bwd_kind<T, BS, HAS_PAD, QM, 0>(a, bhs * (2LL * a.f.n_s + a.f.nb - 2) * (BS / 64), bhs * 2, stream);
}

}  // namespace

extern "C" size_t bb_attn_backward_workspace_bytes(int B, int H, int L, int d, int block) {
  int nb = 0;
  if (check_shape(B, H, L, d, block, 0, &nb) != BB_OK) return 0;
  if (B == 0 || H == 0) return 0;
  return bwd_layout(B, H, L, nb, block).total;
}

extern "C" int bb_attn_backward_ex(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                                   const int32_t* rand_idx, const int32_t* inv_off, const int32_t* inv_rows,
                                   int B, int H, int L, int d, int block, int r, const void* out, const void* dout,
                                   const float* lse, void* dq, void* dk, void* dv, int dtype, void* workspace,
                                   size_t workspace_bytes, void* stream, unsigned flags) {
  if (flags & ~(BB_QUERY_MASK | BB_ORDINARY_UNITS)) return BB_ERR_SHAPE;
  if (dtype != BB_FP32 && dtype != BB_BF16) return BB_ERR_DTYPE;
  int nb = 0;
  const int st = check_shape(B, H, L, d, block, r, &nb);
  if (st != BB_OK) return st;
  if (B == 0 || H == 0) return BB_OK;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !workspace || !inv_off) return BB_ERR_NULL;
  if (r > 0 && (!rand_idx || !inv_rows)) return BB_ERR_NULL;
  const void* a16[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* p : a16)
    if (!aligned(p, 16)) return BB_ERR_ALIGN;
  if ((pad_mask && !aligned(pad_mask, 8)) || !aligned(workspace, 256) || !aligned(lse, 4) ||
      !aligned(inv_off, 4) || (rand_idx && !aligned(rand_idx, 4)) || (inv_rows && !aligned(inv_rows, 4)))
    return BB_ERR_ALIGN;
  const size_t bytes = static_cast<size_t>(B) * H * L * d * (dtype == BB_BF16 ? 2 : 4);
  const void* ins[] = {q, k, v, out, dout};
  for (void* g : {dq, dk, dv}) {
    for (const void* x : ins)
      if (overlap(g, x, bytes)) return BB_ERR_ALIAS;
  }
  if (overlap(dq, dk, bytes) || overlap(dq, dv, bytes) || overlap(dk, dv, bytes)) return BB_ERR_ALIAS;
  const BwdLayout w = bwd_layout(B, H, L, nb, block);
  if (workspace_bytes < w.total) return BB_ERR_WORKSPACE;

  BwdArgs a{};
  a.f.q = static_cast<const char*>(q);
  a.f.k = static_cast<const char*>(k);
  a.f.v = static_cast<const char*>(v);
  a.f.pad = pad_mask;
  a.f.rand_idx = rand_idx;
  a.f.H = H;
  a.f.L = L;
  a.f.nb = nb;
  a.f.r = r;
  a.f.n_s = (nb + kChunkTiles - 1) / kChunkTiles;
  a.f.qmask = (flags & BB_QUERY_MASK) && pad_mask != nullptr ? 1 : 0;
  a.f.gc = a.f.mc = 0;
  if (!(flags & BB_ORDINARY_UNITS)) {
    const SmallSplit sp = bwd_split(B, H, nb, block);
    a.f.gc = sp.gc;
    a.f.mc = sp.mc;
  }
  a.o = static_cast<const char*>(out);
  a.dout = static_cast<const char*>(dout);
  a.lse = lse;
  a.inv_off = inv_off;
  a.inv_rows = inv_rows;
  char* ws = static_cast<char*>(workspace);
  a.rowstat = reinterpret_cast<f32x2*>(ws + w.rowstat);
  a.dq_part = reinterpret_cast<float*>(ws + w.dq);
  a.dk_part = reinterpret_cast<float*>(ws + w.dk);
  a.dv_part = reinterpret_cast<float*>(ws + w.dv);
  a.dq = static_cast<char*>(dq);
  a.dk = static_cast<char*>(dk);
  a.dv = static_cast<char*>(dv);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.f.qmask) {   // pair masking (pad_mask given)
    if (dtype == BB_BF16)
      return block == 64 ? launch_bwd<__bf16, 64, true, true>(a, B, H, s) : launch_bwd<__bf16, 128, true, true>(a, B, H, s);
    return block == 64 ? launch_bwd<float, 64, true, true>(a, B, H, s) : launch_bwd<float, 128, true, true>(a, B, H, s);
  }
  if (dtype == BB_BF16) {
    if (block == 64)
      return pad_mask ? launch_bwd<__bf16, 64, true, false>(a, B, H, s) : launch_bwd<__bf16, 64, false, false>(a, B, H, s);
    return pad_mask ? launch_bwd<__bf16, 128, true, false>(a, B, H, s) : launch_bwd<__bf16, 128, false, false>(a, B, H, s);
  }
  if (block == 64)
    return pad_mask ? launch_bwd<float, 64, true, false>(a, B, H, s) : launch_bwd<float, 64, false, false>(a, B, H, s);
  return pad_mask ? launch_bwd<float, 128, true, false>(a, B, H, s) : launch_bwd<float, 128, false, false>(a, B, H, s);
}

extern "C" int bb_attn_backward(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                                const int32_t* rand_idx, const int32_t* inv_off, const int32_t* inv_rows,
                                int B, int H, int L, int d, int block, int r, const void* out, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, int dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return bb_attn_backward_ex(q, k, v, pad_mask, rand_idx, inv_off, inv_rows, B, H, L, d, block, r, out, dout, lse,
                             dq, dk, dv, dtype, workspace, workspace_bytes, stream, 0u);
}

// --------------------------------------------------------------- layer host --

namespace {

struct LayerLayout {
  size_t q, k, v, o, attn, total;
};

LayerLayout layer_layout(int B, int L, int hidden, int H, int block) {
  const size_t plane = static_cast<size_t>(B) * L * hidden * 2;
  LayerLayout w;
  w.q = 0;
  w.k = w.q + align256(plane);
  w.v = w.k + align256(plane);
  w.o = w.v + align256(plane);
  w.attn = w.o + align256(plane);
  w.total = w.attn + bb_attn_workspace_bytes(B, H, L, kD, block);
  return w;
}

int check_layer(int B, int L, int hidden, int H, int block, int r) {
  if (B < 0 || L <= 0 || H <= 0 || hidden <= 0) return BB_ERR_SHAPE;
  if (hidden != H * kD || hidden % 128 != 0 || L % 128 != 0) return BB_ERR_SHAPE;
  int nb = 0;
  return check_shape(B, H, L, kD, block, r, &nb);
}

}  // namespace

extern "C" size_t bb_layer_workspace_bytes(int B, int L, int hidden, int H, int block) {
  if (check_layer(B, L, hidden, H, block, 0) != BB_OK || B == 0) return 0;
  return layer_layout(B, L, hidden, H, block).total;
}

namespace {

// Checks of one layer's arguments (no HIP call); BB_OK means layer_launch may run.
int layer_check(const void* x, const void* w_qkv, const float* b_qkv, const void* w_o, const float* b_o,
                const uint8_t* pad_mask, const int32_t* rand_idx, int B, int L, int hidden, int H, int block, int r,
                const void* y, int dtype, const void* workspace, size_t workspace_bytes, size_t need) {
  if (dtype != BB_BF16) return BB_ERR_DTYPE;   // the layer runs in bf16 only
  const int st = check_layer(B, L, hidden, H, block, r);
  if (st != BB_OK) return st;
  if (B == 0) return BB_OK;
  if (!x || !w_qkv || !b_qkv || !w_o || !b_o || !y || !workspace) return BB_ERR_NULL;
  if (r > 0 && !rand_idx) return BB_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_qkv, 16) || !aligned(w_o, 16) || !aligned(y, 16) || !aligned(b_qkv, 16) ||
      !aligned(b_o, 16) || !aligned(workspace, 256) || (pad_mask && !aligned(pad_mask, 8)) ||
      (rand_idx && !aligned(rand_idx, 4)))
    return BB_ERR_ALIGN;
  const size_t xbytes = static_cast<size_t>(B) * L * hidden * 2;
  if (overlap(y, x, xbytes)) return BB_ERR_ALIAS;
  if (workspace_bytes < need) return BB_ERR_WORKSPACE;
  return BB_OK;
}

// One layer on `stream` (arguments checked by layer_check): the QKV
// projection into the workspace, the attention, the output projection into y.
int layer_launch(const void* x, const void* w_qkv, const float* b_qkv, const void* w_o, const float* b_o,
                 const uint8_t* pad_mask, const int32_t* rand_idx, int B, int L, int hidden, int H, int block, int r,
                 void* y, char* ws, size_t workspace_bytes, hipStream_t s) {
  const LayerLayout w = layer_layout(B, L, hidden, H, block);
  const int M = B * L;
  ProjArgs pa{};
  pa.a = static_cast<const char*>(x);
  pa.w = static_cast<const char*>(w_qkv);
  pa.bias = b_qkv;
  pa.out = ws + w.q;   // q, k, v planes follow each other (each B*L*hidden*2 bytes, 256-aligned)
  pa.M = M;
  pa.N = 3 * hidden;
  pa.K = hidden;
  pa.L = L;
  pa.H = H;
  pa.hidden = hidden;
  launch_proj<0>(pa, s);
  if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
  const int fst = forward_impl(ws + w.q, ws + w.k, ws + w.v, pad_mask, rand_idx, B, H, L, kD, block, r, ws + w.o,
                               BB_BF16, ws + w.attn, workspace_bytes - w.attn, s, BB_LAUNCH_FUSED, nullptr,
                               nullptr, nullptr);
  if (fst != BB_OK) return fst;
  ProjArgs po = pa;
  po.a = ws + w.o;
  po.w = static_cast<const char*>(w_o);
  po.bias = b_o;
  po.out = static_cast<char*>(y);
  po.N = hidden;
  launch_proj<1>(po, s);
  if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
  return BB_OK;
}

}  // namespace

extern "C" int bb_layer_forward(const void* x, const void* w_qkv, const float* b_qkv, const void* w_o,
                                const float* b_o, const uint8_t* pad_mask, const int32_t* rand_idx, int B, int L,
                                int hidden, int H, int block, int r, void* y, int dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const size_t need = check_layer(B, L, hidden, H, block, r) == BB_OK && B > 0
                          ? layer_layout(B, L, hidden, H, block).total : 0;
  const int st = layer_check(x, w_qkv, b_qkv, w_o, b_o, pad_mask, rand_idx, B, L, hidden, H, block, r, y, dtype,
                             workspace, workspace_bytes, need);
  if (st != BB_OK || B == 0) return st;
  return layer_launch(x, w_qkv, b_qkv, w_o, b_o, pad_mask, rand_idx, B, L, hidden, H, block, r, y,
                      static_cast<char*>(workspace), workspace_bytes, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------- layer stack --

extern "C" size_t bb_layer_stack_workspace_bytes(int B, int L, int hidden, int H, int block) {
  const size_t one = bb_layer_workspace_bytes(B, L, hidden, H, block);
  if (one == 0) return 0;
  return align256(one) + static_cast<size_t>(B) * L * hidden * 2;
}

extern "C" int bb_layer_stack_forward(const void* x, const void* const* w_qkv, const float* const* b_qkv,
                                      const void* const* w_o, const float* const* b_o, const uint8_t* pad_mask,
                                      const int32_t* const* rand_idx, int n_layers, int B, int L, int hidden,
                                      int H, int block, int r, void* y, int dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (n_layers < 0) return BB_ERR_SHAPE;
  if (dtype != BB_BF16) return BB_ERR_DTYPE;   // the layer runs in bf16 only
  int st = check_layer(B, L, hidden, H, block, r);
  if (st != BB_OK) return st;
  if (B == 0 || n_layers == 0) return n_layers == 0 && B > 0 ? BB_ERR_SHAPE : BB_OK;
  if (!w_qkv || !b_qkv || !w_o || !b_o || (r > 0 && !rand_idx)) return BB_ERR_NULL;
  const size_t one = layer_layout(B, L, hidden, H, block).total;
  const size_t act_off = align256(one);
  const size_t need = act_off + static_cast<size_t>(B) * L * hidden * 2;
  if (workspace == nullptr) return BB_ERR_NULL;
  char* act = static_cast<char*>(workspace) + act_off;   // the activations between layers
  // layer l writes y when n_layers - 1 - l is even, else act: the last layer
  // writes y and consecutive layers alternate
  auto out_of = [&](int l) -> void* { return ((n_layers - 1 - l) & 1) == 0 ? y : static_cast<void*>(act); };
  for (int l = 0; l < n_layers; ++l) {   // every check before the first launch
    const void* in = l == 0 ? x : out_of(l - 1);
    st = layer_check(in, w_qkv[l], b_qkv[l], w_o[l], b_o[l], pad_mask, r > 0 ? rand_idx[l] : nullptr, B, L,
                     hidden, H, block, r, out_of(l), dtype, workspace, workspace_bytes, need);
    if (st != BB_OK) return st;
  }
  const size_t xbytes = static_cast<size_t>(B) * L * hidden * 2;
  if (overlap(y, x, xbytes) || overlap(workspace, need, x, xbytes) || overlap(workspace, need, y, xbytes))
    return BB_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int l = 0; l < n_layers; ++l) {
    st = layer_launch(l == 0 ? x : out_of(l - 1), w_qkv[l], b_qkv[l], w_o[l], b_o[l], pad_mask,
                      r > 0 ? rand_idx[l] : nullptr, B, L, hidden, H, block, r, out_of(l),
                      static_cast<char*>(workspace), one, s);
    if (st != BB_OK) return st;
  }
  return BB_OK;
}
