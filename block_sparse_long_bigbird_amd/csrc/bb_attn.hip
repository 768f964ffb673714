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
//     partial (row max, row sum, O) and the last unit of its block to arrive
//     merges all partials in fixed chunk order (deterministic).
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
// PV MFMA wants.  V is staged transposed in LDS (V^T, dims x keys).
// The two key-half waves of a query group merge their (max, sum, O) states
// through LDS at the end.
//
// fp32 inputs run the same code with fp32 MFMA (32x32x2) and fp32 P.

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "bb_attn.h"

namespace {

constexpr int kD = 64;                   // supported head dimension
constexpr int kChunkTiles = 8;           // key tiles per global-row work unit
constexpr int kMaxR = 16;                // random blocks per row, upper bound
constexpr int kMaxTiles = 5 + kMaxR;     // longest tile list of a unit
constexpr float kScaleLog2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
constexpr float kMaskRaw = -10000.0f * 8.0f;  // -10000 on the logit, in q.k units
constexpr float kRescaleTau = 8.0f;      // lazy rescale threshold (log2 units)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T, int BS>
struct Cfg {
  static constexpr int ES = sizeof(T);
  static constexpr int EPC = 16 / ES;           // elements per 16-byte chunk
  static constexpr int CPR_K = kD * ES / 16;    // chunks per K row in LDS (and per Q/V row)
  static constexpr int CPR_V = BS * ES / 16;    // chunks per V^T row in LDS
  static constexpr int WQ = BS / 32;            // query groups
  static constexpr int WK = 2;                  // key halves
  static constexpr int NW = WQ * WK;            // waves per workgroup
  static constexpr int NT = 64 * NW;            // threads per workgroup
  static constexpr int NSUB = BS / (32 * WK);   // 32-key subtiles per wave per tile
  static constexpr int K_BYTES = BS * kD * ES;
  static constexpr int STAGE = 2 * K_BYTES;     // K tile + V^T tile
  static constexpr int K_TASKS = BS * CPR_K / NT;        // K chunks per thread per tile
  static constexpr int V_TASKS = (BS / 2) * CPR_K / NT;  // V row-pair chunks per thread
  static constexpr int QC = CPR_K / 2;          // Q chunks per lane
  static constexpr int MERGE_BYTES = WQ * 34 * 64 * 4;
  static constexpr int SMEM = (2 * STAGE > MERGE_BYTES ? 2 * STAGE : MERGE_BYTES);
  static_assert(K_TASKS * NT == BS * CPR_K, "K staging must tile evenly");
  static_assert(V_TASKS * NT == (BS / 2) * CPR_K, "V staging must tile evenly");
  static_assert(NSUB >= 1, "at least one subtile per wave");
  static_assert(CPR_V % 8 == 0 && CPR_K % 8 == 0, "swizzle needs 8-chunk groups");
};

struct Args {
  const char* q;
  const char* k;
  const char* v;
  const uint8_t* pad;
  const int32_t* rand_idx;
  char* out;
  uint32_t* ctr;   // [B*H][2] arrival counters
  float* pm;       // [B*H][2][n_s][BS] partial row max (q.k units)
  float* pl;       // [B*H][2][n_s][BS] partial row sum
  float* po;       // [B*H][2][n_s][BS][kD] partial unnormalised output
  int H, L, nb, r, n_s;
};

// 16-byte LDS chunk swizzle.  A wave reads rows perm_row(0..31) (+ a multiple
// of 32) at one logical chunk; the 8 lanes served together hit rows
// {R..R+3, R+8..R+11}, which this XOR spreads over 8 distinct chunk slots.
__device__ __forceinline__ int swz(int row) { return (row & 3) | ((row >> 1) & 4); }

// MFMA row i (0..31) -> key / dim offset inside a 32-wide subtile, chosen so
// that accumulator register v of lane group g holds offset
// 16*(v/8) + 8*g + (v%8): two runs of 8 consecutive keys per lane.
__device__ __forceinline__ int perm_row(int i) {
  const int a = i >> 3, gg = (i >> 2) & 1, c = i & 3;
  return 16 * (a >> 1) + 8 * gg + 4 * (a & 1) + c;
}

// XCD-aware work order: hardware hands consecutive workgroup ids to the 8 XCDs
// round robin; remap so each XCD runs a contiguous range of work units (one
// (batch, head) after another), which keeps that unit's K/V in its own L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, rem = n & 7, x = bid & 7, k = bid >> 3;
  return x * q + (x < rem ? x : rem) + k;
}

__device__ __forceinline__ bool has_zero_byte(uint64_t x) {
  return ((x - 0x0101010101010101ull) & ~x & 0x8080808080808080ull) != 0;
}

template <typename T, int BS>
struct StageRegs {
  u32x4 k[Cfg<T, BS>::K_TASKS];
  u32x4 v0[Cfg<T, BS>::V_TASKS];
  u32x4 v1[Cfg<T, BS>::V_TASKS];
  u32x4 pad;
};

// Global -> registers for key tile `tile` of (b, h).
template <typename T, int BS>
__device__ __forceinline__ void load_tile(StageRegs<T, BS>& st, const char* kbh, const char* vbh,
                                          const uint8_t* pad_b, int tile, int tid) {
  using C = Cfg<T, BS>;
  constexpr int ROWB = kD * C::ES;
  const char* kt = kbh + static_cast<size_t>(tile) * BS * ROWB;
  const char* vt = vbh + static_cast<size_t>(tile) * BS * ROWB;
#pragma unroll
  for (int t = 0; t < C::K_TASKS; ++t) {
    const int task = tid + C::NT * t;
    const int row = task / C::CPR_K, c = task % C::CPR_K;
    st.k[t] = *reinterpret_cast<const u32x4*>(kt + row * ROWB + c * 16);
  }
#pragma unroll
  for (int t = 0; t < C::V_TASKS; ++t) {
    const int task = tid + C::NT * t;
    const int dc = task % C::CPR_K, kp = task / C::CPR_K;
    st.v0[t] = *reinterpret_cast<const u32x4*>(vt + (2 * kp) * ROWB + dc * 16);
    st.v1[t] = *reinterpret_cast<const u32x4*>(vt + (2 * kp + 1) * ROWB + dc * 16);
  }
  if (pad_b != nullptr && tid < BS / 16)
    st.pad = *reinterpret_cast<const u32x4*>(pad_b + static_cast<size_t>(tile) * BS + tid * 16);
}

// Registers -> LDS stage: K as [key][dim], V transposed as [dim][key].
template <typename T, int BS>
__device__ __forceinline__ void store_tile(const StageRegs<T, BS>& st, char* sb, uint8_t* spad,
                                           bool has_pad, int tid) {
  using C = Cfg<T, BS>;
#pragma unroll
  for (int t = 0; t < C::K_TASKS; ++t) {
    const int task = tid + C::NT * t;
    const int row = task / C::CPR_K, c = task % C::CPR_K;
    *reinterpret_cast<u32x4*>(sb + (row * C::CPR_K + (c ^ swz(row))) * 16) = st.k[t];
  }
  char* vt = sb + C::K_BYTES;
#pragma unroll
  for (int t = 0; t < C::V_TASKS; ++t) {
    const int task = tid + C::NT * t;
    const int dc = task % C::CPR_K, kp = task / C::CPR_K;
    const int key = 2 * kp;
    const int ck = key / C::EPC;                 // chunk of the key pair in a V^T row
    const int off = (key % C::EPC) * C::ES;      // byte offset of the pair in that chunk
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = st.v0[t][w], b = st.v1[t][w];
        const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05040100u);  // (a.lo, b.lo)
        const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07060302u);  // (a.hi, b.hi)
        const int d0 = dc * 8 + 2 * w, d1 = d0 + 1;
        *reinterpret_cast<uint32_t*>(vt + (d0 * C::CPR_V + (ck ^ swz(d0))) * 16 + off) = lo;
        *reinterpret_cast<uint32_t*>(vt + (d1 * C::CPR_V + (ck ^ swz(d1))) * 16 + off) = hi;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dd = dc * 4 + e;
        f32x2 pr = {__uint_as_float(st.v0[t][e]), __uint_as_float(st.v1[t][e])};
        *reinterpret_cast<f32x2*>(vt + (dd * C::CPR_V + (ck ^ swz(dd))) * 16 + off) = pr;
      }
    }
  }
  if (has_pad && tid < BS / 16) *reinterpret_cast<u32x4*>(spad + tid * 16) = st.pad;
}

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

// Per-wave online-softmax state for 32 query rows (one per lane pair).
struct WaveState {
  f32x16 o[2];   // O^T, dims [0,32) and [32,64)
  float m;       // running row max in q.k units (may lag the true max by < tau/scale)
  float l;       // this lane's part of the row sum
};

// One 32-key subtile: scores, online softmax, PV.
template <typename T, int BS>
__device__ __forceinline__ void subtile(WaveState& ws, const u32x4 (&qop)[Cfg<T, BS>::QC],
                                        const char* sb, const uint8_t* spad, bool has_pad,
                                        int kbase, int j, int g) {
  using C = Cfg<T, BS>;
  // ---- S^T = K . Q^T (+ key bias) -------------------------------------------
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  if (has_pad) {
    const uint64_t w0 = *reinterpret_cast<const uint64_t*>(spad + kbase + 8 * g);
    const uint64_t w1 = *reinterpret_cast<const uint64_t*>(spad + kbase + 16 + 8 * g);
    if (__any(has_zero_byte(w0) || has_zero_byte(w1))) {
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        acc[v] = ((w0 >> (8 * v)) & 0xffu) ? 0.0f : kMaskRaw;
        acc[8 + v] = ((w1 >> (8 * v)) & 0xffu) ? 0.0f : kMaskRaw;
      }
    }
  }
  {
    const int row = kbase + perm_row(j);
    const int sw = swz(row);
#pragma unroll
    for (int x = 0; x < C::QC; ++x) {
      const int c = 2 * x + g;
      const u32x4 a = *reinterpret_cast<const u32x4*>(sb + (row * C::CPR_K + (c ^ sw)) * 16);
      acc = mfma_qk(a, qop[x], acc, static_cast<T*>(nullptr));
    }
  }
  // ---- online softmax (lane = query row; 16 of its 32 keys) ----------------
  float mloc = acc[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) mloc = fmaxf(mloc, acc[v]);
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  const float m_new = fmaxf(ws.m, mloc);
  if (__any((m_new - ws.m) * kScaleLog2 > kRescaleTau)) {
    const float alpha = __builtin_amdgcn_exp2f((ws.m - m_new) * kScaleLog2);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      ws.o[0][v] *= alpha;
      ws.o[1][v] *= alpha;
    }
    ws.l *= alpha;
    ws.m = m_new;
  }
  const float mc = ws.m * kScaleLog2;
  float p[16];
  float lsum = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kScaleLog2, -mc));
    lsum += p[v];
  }
  ws.l += lsum;
  // ---- O^T += V^T . P^T -------------------------------------------------------
  const char* vt = sb + C::K_BYTES;
  if constexpr (sizeof(T) == 2) {
    bf16x8 pb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        f32x2 pr = {p[8 * h + e], p[8 * h + e + 1]};
        bf16x2 c2 = __builtin_convertvector(pr, bf16x2);
        pb[h][e] = c2[0];
        pb[h][e + 1] = c2[1];
      }
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const int row = dh * 32 + perm_row(j);
      const int sw = swz(row);
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int c = kbase / 8 + 2 * mm + g;
        const u32x4 a = *reinterpret_cast<const u32x4*>(vt + (row * C::CPR_V + (c ^ sw)) * 16);
        ws.o[dh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[mm],
                                                           ws.o[dh], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const int row = dh * 32 + perm_row(j);
      const int sw = swz(row);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = kbase / 4 + 4 * (q4 >> 1) + 2 * g + (q4 & 1);
        const f32x4 a = *reinterpret_cast<const f32x4*>(vt + (row * C::CPR_V + (c ^ sw)) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ws.o[dh] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], p[4 * q4 + e], ws.o[dh], 0, 0, 0);
      }
    }
  }
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
  f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
  reinterpret_cast<f32x4*>(dst)[0] = a;
  reinterpret_cast<f32x4*>(dst)[1] = b;
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


// One work unit on (b, h).  gsel < 0: middle query block qb, finalised in
// place.  gsel in {0, 1}: global query block qb (0 or nb-1), key chunk
// `chunk` of split-K; the last chunk to arrive merges all partials.
template <typename T, int BS>
__device__ __forceinline__ void run_unit(const Args& a, int b, int h, int qb, int gsel, int chunk) {
  using C = Cfg<T, BS>;
  constexpr int ROWB = kD * C::ES;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ __attribute__((aligned(16))) uint8_t spad[2][BS];
  __shared__ int s_tiles[kMaxTiles];
  __shared__ int s_last;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wq = wave % C::WQ, wk = wave / C::WQ;
  const int j = lane & 31, g = lane >> 5;
  const int nb = a.nb, L = a.L;
  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const char* qbh = a.q + bh * L * ROWB;
  const char* kbh = a.k + bh * L * ROWB;
  const char* vbh = a.v + bh * L * ROWB;
  const bool has_pad = a.pad != nullptr;
  const uint8_t* pad_b = has_pad ? a.pad + static_cast<size_t>(b) * L : nullptr;

  // ---- key-tile list --------------------------------------------------------
  int ntiles;
  if (gsel < 0) {
    const int lo = qb - 1 < 1 ? 1 : qb - 1;            // band without the global blocks
    const int hi = qb + 1 > nb - 2 ? nb - 2 : qb + 1;
    ntiles = 2 + (hi - lo + 1) + a.r;
    if (tid == 0) {
      int n = 0;
      s_tiles[n++] = 0;
      for (int t = lo; t <= hi; ++t) s_tiles[n++] = t;
      s_tiles[n++] = nb - 1;
      const int32_t* rr = a.rand_idx + (static_cast<size_t>(h) * (nb - 2) + (qb - 1)) * a.r;
      for (int t = 0; t < a.r; ++t) {
        int e = rr[t];
        e = e < 1 ? 1 : (e > nb - 2 ? nb - 2 : e);    // never read outside the sequence
        s_tiles[n++] = e;
      }
    }
  } else {
    const int t0 = chunk * kChunkTiles;
    ntiles = nb - t0 < kChunkTiles ? nb - t0 : kChunkTiles;
    if (tid < ntiles) s_tiles[tid] = t0 + tid;
  }

  // ---- this wave's 32 query rows as the B operand of the score MFMA --------
  const int q0 = qb * BS + wq * 32;
  u32x4 qop[C::QC];
  {
    const char* qrow = qbh + static_cast<size_t>(q0 + j) * ROWB;
#pragma unroll
    for (int x = 0; x < C::QC; ++x) qop[x] = *reinterpret_cast<const u32x4*>(qrow + (2 * x + g) * 16);
  }

  WaveState ws;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    ws.o[0][v] = 0.0f;
    ws.o[1][v] = 0.0f;
  }
  ws.m = -__builtin_inff();
  ws.l = 0.0f;

  // ---- double-buffered tile loop ---------------------------------------------
  __syncthreads();
  StageRegs<T, BS> st;
  load_tile<T, BS>(st, kbh, vbh, pad_b, s_tiles[0], tid);
  store_tile<T, BS>(st, smem, spad[0], has_pad, tid);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) load_tile<T, BS>(st, kbh, vbh, pad_b, s_tiles[t + 1], tid);
    const char* sb = smem + cur * C::STAGE;
#pragma unroll
    for (int s = 0; s < C::NSUB; ++s)
      subtile<T, BS>(ws, qop, sb, spad[cur], has_pad, wk * (BS / 2) + 32 * s, j, g);
    if (t + 1 < ntiles) store_tile<T, BS>(st, smem + (cur ^ 1) * C::STAGE, spad[cur ^ 1], has_pad, tid);
    __syncthreads();
  }

  // ---- merge the two key halves of each query group ------------------------
  float* mrg = reinterpret_cast<float*>(smem) + wq * 34 * 64;
  if (wk == 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      mrg[v * 64 + lane] = ws.o[0][v];
      mrg[(16 + v) * 64 + lane] = ws.o[1][v];
    }
    mrg[32 * 64 + lane] = ws.m;
    mrg[33 * 64 + lane] = ws.l;
  }
  __syncthreads();
  if (wk == 0) {
    const float m1 = mrg[32 * 64 + lane], l1 = mrg[33 * 64 + lane];
    const float mm = fmaxf(ws.m, m1);
    const float a0 = __builtin_amdgcn_exp2f((ws.m - mm) * kScaleLog2);
    const float a1 = __builtin_amdgcn_exp2f((m1 - mm) * kScaleLog2);
    float o[2][16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      o[0][v] = ws.o[0][v] * a0 + mrg[v * 64 + lane] * a1;
      o[1][v] = ws.o[1][v] * a0 + mrg[(16 + v) * 64 + lane] * a1;
    }
    float l = ws.l * a0 + l1 * a1;
    l += __shfl_xor(l, 32);
    if (gsel < 0) {
      char* orow = a.out + (bh * L + q0 + j) * ROWB;
      const float inv = 1.0f / l;
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = o[dh][8 * h8 + e] * inv;
          store_row8(orow + (dh * 32 + 16 * h8 + 8 * g) * C::ES, x, static_cast<T*>(nullptr));
        }
    } else {
      const size_t pidx = ((bh * 2 + gsel) * a.n_s + chunk) * BS + wq * 32 + j;
      char* prow = reinterpret_cast<char*>(a.po + pidx * kD);
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8)
          store_row8(prow + (dh * 32 + 16 * h8 + 8 * g) * 4, &o[dh][8 * h8], static_cast<float*>(nullptr));
      if (g == 0) {
        a.pm[pidx] = mm;
        a.pl[pidx] = l;
      }
    }
  }
  if (gsel < 0) return;

  // ---- split-K: the last chunk of this global block merges all partials -----
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.ctr + bh * 2 + gsel, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == static_cast<unsigned>(a.n_s - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const size_t base = (bh * 2 + gsel) * a.n_s;
  for (int idx = tid; idx < BS * kD / 4; idx += C::NT) {
    const int ql = idx / (kD / 4), dq = idx % (kD / 4);
    float mx = -__builtin_inff();
    for (int s = 0; s < a.n_s; ++s) mx = fmaxf(mx, a.pm[(base + s) * BS + ql]);
    f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f;
    for (int s = 0; s < a.n_s; ++s) {              // fixed order: deterministic
      const size_t pi = (base + s) * BS + ql;
      const float w = __builtin_amdgcn_exp2f((a.pm[pi] - mx) * kScaleLog2);
      den += w * a.pl[pi];
      const f32x4 po = *reinterpret_cast<const f32x4*>(a.po + pi * kD + dq * 4);
      num += w * po;
    }
    const float inv = 1.0f / den;
    store_f32x4(a.out + (bh * L + static_cast<size_t>(qb) * BS + ql) * ROWB + dq * 4 * C::ES,
                num * inv, static_cast<T*>(nullptr));
  }
  if (tid == 0) __hip_atomic_store(a.ctr + bh * 2 + gsel, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Decode a work unit.  Per (b, h): 2*n_s global units (block 0 chunks, then
// block nb-1 chunks) followed by nb-2 middle units.  kind selects which of
// them this grid covers: 0 = all, 1 = global units only, 2 = middle only.
template <typename T, int BS, int kind>
__device__ __forceinline__ void dispatch(const Args& a) {
  const int n_g = kind == 2 ? 0 : 2 * a.n_s;
  const int n_m = kind == 1 ? 0 : a.nb - 2;
  const int per_bh = n_g + n_m;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = unit / per_bh, u = unit % per_bh;
  const int b = bh / a.H, h = bh % a.H;
  int qb, gsel, chunk;
  if (u < n_g) {
    gsel = u / a.n_s;
    chunk = u % a.n_s;
    qb = gsel ? a.nb - 1 : 0;
  } else {
    gsel = -1;
    chunk = 0;
    qb = u - n_g + 1;
  }
  run_unit<T, BS>(a, b, h, qb, gsel, chunk);
}

template <typename T, int BS>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) bb_fused_kernel(Args a) {
  dispatch<T, BS, 0>(a);
}
template <typename T, int BS>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) bb_global_rows_kernel(Args a) {
  dispatch<T, BS, 1>(a);
}
template <typename T, int BS>
__global__ void __launch_bounds__((Cfg<T, BS>::NT)) bb_middle_rows_kernel(Args a) {
  dispatch<T, BS, 2>(a);
}

// ---------------------------------------------------------------- host side --

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
  size_t ctr, pm, pl, po, total;
};

Layout workspace_layout(int B, int H, int nb, int block) {
  const size_t n_s = static_cast<size_t>((nb + kChunkTiles - 1) / kChunkTiles);
  const size_t units = static_cast<size_t>(B) * H * 2;
  Layout w;
  w.ctr = 0;
  w.pm = align256(units * sizeof(uint32_t));
  w.pl = w.pm + align256(units * n_s * block * sizeof(float));
  w.po = w.pl + align256(units * n_s * block * sizeof(float));
  w.total = w.po + units * n_s * block * kD * sizeof(float);
  return w;
}

int check_shape(int B, int H, int L, int d, int block, int r, int* nb_out) {
  if (B < 0 || H < 0 || L <= 0 || r < 0) return BB_ERR_SHAPE;
  if (d != kD) return BB_ERR_SHAPE;
  if (block != 64 && block != 128) return BB_ERR_SHAPE;
  if (L % block != 0) return BB_ERR_SHAPE;
  const int nb = L / block;
  if (nb < 3) return BB_ERR_SHAPE;
  const int r_max = nb - 5 > 0 ? nb - 5 : 0;
  if (r > r_max || r > kMaxR) return BB_ERR_SHAPE;
  const int n_s = (nb + kChunkTiles - 1) / kChunkTiles;
  const long long units = static_cast<long long>(B) * H * (2LL * n_s + nb - 2);
  if (units > 0x7fffffffLL) return BB_ERR_SHAPE;
  *nb_out = nb;
  return BB_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

template <typename T, int BS>
int launch(const Args& a, int B, int H, hipStream_t stream, unsigned flags) {
  using C = Cfg<T, BS>;
  const int per_g = 2 * a.n_s, per_m = a.nb - 2;
  const unsigned bhs = static_cast<unsigned>(B) * static_cast<unsigned>(H);
  if (flags == BB_LAUNCH_SPLIT) {
    bb_global_rows_kernel<T, BS><<<dim3(bhs * per_g), dim3(C::NT), 0, stream>>>(a);
    if (hipGetLastError() != hipSuccess) return BB_ERR_HIP;
    bb_middle_rows_kernel<T, BS><<<dim3(bhs * per_m), dim3(C::NT), 0, stream>>>(a);
  } else {
    bb_fused_kernel<T, BS><<<dim3(bhs * (per_g + per_m)), dim3(C::NT), 0, stream>>>(a);
  }
  return hipGetLastError() == hipSuccess ? BB_OK : BB_ERR_HIP;
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

extern "C" size_t bb_attn_workspace_bytes(int B, int H, int L, int d, int block) {
  int nb = 0;
  if (check_shape(B, H, L, d, block, 0, &nb) != BB_OK) return 0;
  if (B == 0 || H == 0) return 0;
  return workspace_layout(B, H, nb, block).total;
}

extern "C" int bb_attn_forward_ex(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                                  const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                                  void* out, int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream, unsigned flags) {
  if (dtype != BB_FP32 && dtype != BB_BF16) return BB_ERR_DTYPE;
  if (flags != BB_LAUNCH_FUSED && flags != BB_LAUNCH_SPLIT) return BB_ERR_SHAPE;
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
  a.ctr = reinterpret_cast<uint32_t*>(ws + w.ctr);
  a.pm = reinterpret_cast<float*>(ws + w.pm);
  a.pl = reinterpret_cast<float*>(ws + w.pl);
  a.po = reinterpret_cast<float*>(ws + w.po);
  a.H = H;
  a.L = L;
  a.nb = nb;
  a.r = r;
  a.n_s = (nb + kChunkTiles - 1) / kChunkTiles;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == BB_BF16)
    return block == 64 ? launch<__bf16, 64>(a, B, H, s, flags) : launch<__bf16, 128>(a, B, H, s, flags);
  return block == 64 ? launch<float, 64>(a, B, H, s, flags) : launch<float, 128>(a, B, H, s, flags);
}

extern "C" int bb_attn_forward(const void* q, const void* k, const void* v, const uint8_t* pad_mask,
                               const int32_t* rand_idx, int B, int H, int L, int d, int block, int r,
                               void* out, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return bb_attn_forward_ex(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, dtype, workspace,
                            workspace_bytes, stream, BB_LAUNCH_FUSED);
}
