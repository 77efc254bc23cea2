// Device-side building blocks shared by the gfx950 (CDNA4) kernels of
// block-diffusion attention: element types and MFMA wrappers, operand reads
// from swizzled LDS tiles, tile copies straight into LDS, and the waits that
// go with them.
//
// MFMA 32x32 operand and result layout (lane l of a 64-lane wave):
//   A (32 x 16): row l%32, 8 contraction slots; B (16 x 32): column l%32,
//   8 slots. The hardware pairs slot j of A with slot j of B for the same
//   lane half h = l/32; which contraction index a slot stands for is the
//   caller's choice as long as A and B agree. Here slot j of half h in the
//   16-deep step starting at k0 stands for k0 + 8h + j ("natural"), or, when an
//   operand is built from a result tile, for k0 + 8(j/4) + 4h + j%4 ("result
//   order").
//   C (32 x 32, 16 floats): column l%32, element i is row 8(i/4) + 4h + i%4.
//
// LDS tiles are row-major with no padding; the 16-byte chunk c of row r sits
// at chunk position c ^ swz(r), swz(r) = 4(r%4) + (r/4)%4. The LDS has 64
// banks: a row-slice operand read (ds_read_b128, 16 lanes per cycle = 16
// consecutive rows, same chunk) and a transposed operand read
// (ds_read_b64_tr_b16, 32 lanes per cycle = 4 consecutive rows x 64 bytes)
// both hit 64 distinct banks. The transposed read gives lane i of each 16-lane
// group column i of four consecutive rows, i.e. the operand of a matrix whose
// contraction index runs down the tile's rows, so no transposed copy is ever
// stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bdattn_mask.h"
#include "launch.h"

namespace bdattn {
namespace dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float floatx2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short shortx4;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

template <int N>
using Int = std::integral_constant<int, N>;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The forward moves its running row maximum (log2 units) as soon as a tile's
// maximum exceeds it, so the largest softmax weight of a row is exactly 1
// when it is rounded to bf16 for the P V product. (Letting the maximum lag by
// a margin saves rescales but rounds the dominant weight, which the gradients
// of strongly peaked rows amplify.)
constexpr float kRescaleMargin = 0.f;

// The work item of this workgroup (the protocol is described with
// kClaimQueues in plan.h): with ctr == nullptr item blockIdx.x of a grid of n;
// else thread 0 claims one (claim_next) from the counters
// ctr[0..kClaimQueues) of a grid of n + claim_extra(n), starting with queue
// blockIdx.x mod 8, and the workgroup reads it from LDS; -1 when every queue
// is empty (the workgroup then ends).
__device__ __forceinline__ int claim_item(int32_t* ctr, int n) {
  __shared__ int s_item;
  if (ctr == nullptr) return blockIdx.x;
  if (threadIdx.x == 0)
    s_item = claim_next(
        blockIdx.x % kClaimQueues, n,
        [&](int y) { return __hip_atomic_load(ctr + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); },
        [&](int y) { return __hip_atomic_fetch_add(ctr + y, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); });
  __syncthreads();
  // (the same in every lane: as a scalar, the work item's fields load into
  // scalar registers and the code that decodes them stays scalar)
  return __builtin_amdgcn_readfirstlane(s_item);
}

// 2^x with one v_exp_f32 (results below 2^-126 flush to zero, which is
// harmless for softmax weights; exp2(-inf) = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Chunk swizzle of row r in a tile with NCH 16-byte chunks per row.
template <int NCH>
__device__ __forceinline__ int tile_swz(int r) {
  return (((r & 3) << 2) | ((r >> 2) & 3)) & (NCH - 1);
}

// Element offset of (row r, column col) in a swizzled tile of D-element rows
// with EPC elements per 16-byte chunk.
template <int D, int EPC>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * D + (((col / EPC) ^ tile_swz<D / EPC>(r)) * EPC) + (col % EPC);
}

// ----------------------------------------------------------------- elements
template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  using T = uint16_t;  // bf16 bits
  static constexpr int EPC = 8;
  struct Frag {
    uint4 v;
  };
  static __device__ __forceinline__ Frag zero() { return Frag{make_uint4(0, 0, 0, 0)}; }
  // 8 consecutive elements from global memory
  static __device__ __forceinline__ Frag load(const T* p) { return Frag{*(const uint4*)p}; }
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    floatx2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
  // 8 floats -> 8 bf16 (round to nearest even)
  static __device__ __forceinline__ Frag pack(const float* x) {
    return Frag{make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]),
                           pack2(x[6], x[7]))};
  }
  static __device__ __forceinline__ float to_f(T v) { return __uint_as_float(uint32_t(v) << 16); }
  static __device__ __forceinline__ T from_f(float x) { return T(pack2(x, 0.f) & 0xffffu); }
  static __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    *(uint2*)p = make_uint2(pack2(a, b), pack2(c, d));
  }
};

template <>
struct Elem<false> {
  using T = float;
  static constexpr int EPC = 4;
  struct Frag {
    float4 a, b;
  };
  static __device__ __forceinline__ Frag zero() {
    return Frag{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)};
  }
  static __device__ __forceinline__ Frag load(const T* p) {
    return Frag{*(const float4*)p, *(const float4*)(p + 4)};
  }
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a.x, b.a.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a.y, b.a.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a.z, b.a.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a.w, b.a.w, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b.x, b.b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b.y, b.b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b.z, b.b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b.w, b.b.w, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag pack(const float* x) {
    return Frag{make_float4(x[0], x[1], x[2], x[3]), make_float4(x[4], x[5], x[6], x[7])};
  }
  static __device__ __forceinline__ float to_f(T v) { return v; }
  static __device__ __forceinline__ T from_f(float x) { return x; }
  static __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    *(float4*)p = make_float4(a, b, c, d);
  }
};

// Per-lane byte offsets of the operand reads from swizzled LDS tiles. The
// swizzle depends on a row's low 4 bits only, so 32-row blocks and 16-row
// steps add compile-time constants to a few offsets fixed per lane. Offsets
// are relative to the start of the kernel's LDS array; the template argument
// TILE of the reads adds the (compile-time) byte offset of the tile itself,
// buffer included.
template <bool BF16, int D>
struct OperandReads {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Frag = typename E::Frag;
  static constexpr int EPC = E::EPC;
  static constexpr uint32_t ROW = D * sizeof(T);  // bytes per tile row
  static constexpr int NCHF = BF16 ? 1 : 2;       // 16-byte chunks per fragment
  static constexpr int NTR = BF16 ? 2 : 8;         // reads per transposed fragment
  uint32_t row[D / 16][NCHF];  // row lane%32, column 16 ks + 8 (lane/32) (+4)
  uint32_t tr[D / 32][NTR];    // transposed: see tr_frag

  __device__ __forceinline__ void init(int lane) {
    const int lq = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int c = 0; c < NCHF; ++c)
        row[ks][c] = sizeof(T) * tile_off<D, EPC>(lq, 16 * ks + 8 * h + 4 * c);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      if (BF16) {
        // ds_read_b64_tr_b16: lanes r/4 = 0..3 of each 16-lane group address
        // four consecutive rows, 4 r%4 columns apart (see the file header)
        const int r = lane & 15, c = (lane >> 4) & 1;
        const int col = 32 * db + 16 * c + 4 * (r & 3);
#pragma unroll
        for (int t = 0; t < NTR; ++t)
          tr[db][t] = sizeof(T) * tile_off<D, EPC>(8 * t + 4 * h + (r >> 2), col);
      } else {
#pragma unroll
        for (int j = 0; j < NTR; ++j)
          tr[db][j] = sizeof(T) * tile_off<D, EPC>(8 * (j >> 2) + 4 * h + (j & 3), 32 * db + lq);
      }
    }
  }
  // 8 consecutive elements of row 32 mb + lane%32, from column 16 ks + 8
  // (lane/32), of the tile TILE bytes into the LDS array `lds`.
  template <uint32_t TILE>
  __device__ __forceinline__ Frag row_frag(const void* lds, int mb, int ks) const {
    const char* b = (const char*)lds + TILE + mb * 32 * ROW;
    if constexpr (BF16) {
      return Frag{*(const uint4*)(b + row[ks][0])};
    } else {
      return Frag{*(const float4*)(b + row[ks][0]), *(const float4*)(b + row[ks][1])};
    }
  }
  // Operand whose contraction index runs down the tile rows, in result order:
  // lane l takes column 32 db + l%32; slot j of half h takes row
  // k0 + 8 (j/4) + 4 h + j%4 (k0 a multiple of 16).
  template <uint32_t TILE>
  __device__ __forceinline__ Frag tr_frag(const void* lds, int k0, int db) const {
    const char* b = (const char*)lds + TILE + k0 * ROW;
    if constexpr (BF16) {
      const shortx4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(b + tr[db][0]));
      const shortx4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(b + tr[db][1]));
      const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
      return Frag{make_uint4(ux.x, ux.y, uy.x, uy.y)};
    } else {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = *(const float*)(b + tr[db][j]);
      return E::pack(x);
    }
  }
};

// Row bounds of local rows of a query stream (0 clean, 1 corrupted), in
// terms of the keys present (clean buffer indices and local corrupted keys),
// from this description of the problem.
struct RowSpace {
  int32_t clean_q_start, B;
  const int32_t* ids;
  bool token_causal;
  int32_t kv0, nkv;  // the clean buffer holds global positions [kv0, kv0 + nkv)
  bool corr_keys;    // the local corrupted keys are present
  const BdDocSpan* docs;  // document of each global block (nullptr: one document)
};
// Bounds of three rows of one stream at once. Every table load (block ids,
// then documents) is issued before any is used, so their round trips overlap
// (a work item's start waits on them).
__device__ __forceinline__ void row_bounds3(int stream, const int32_t (&row)[3], const RowSpace& rs,
                                            BdRowBounds (&out)[3]) {
  int32_t id[3] = {0, 0, 0};
  if (stream) {
#pragma unroll
    for (int i = 0; i < 3; ++i) id[i] = rs.ids[row[i] / rs.B];
  }
  BdDocSpan sp[3];
  if (rs.docs) {  // the document of the row's block (a corrupted row's: its id's)
#pragma unroll
    for (int i = 0; i < 3; ++i) sp[i] = rs.docs[stream == 0 ? (rs.clean_q_start + row[i]) / rs.B : id[i]];
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    BdRowBounds r = stream == 0 ? bd_clean_row(rs.clean_q_start + row[i], rs.B, rs.token_causal)
                                : bd_corr_row(row[i], id[i], rs.B);
    if (rs.docs) r = bd_in_document(r, sp[i]);
    out[i] = bd_in_buffer(r, rs.kv0, rs.nkv, rs.corr_keys);
  }
}

// Buffer rows of the clean key tiles of a gathered buffer: map[j] is the
// buffer tile of key tile j in position order. Tiles are asked for in
// increasing order. Lane i holds the entry of tile base + i, refilled every
// 64 tiles, so a lookup is a register read (v_readlane) except at a refill,
// whose load is lane-varying and so a vector load.
template <int TK>
struct KeyTileMap {
  const int32_t* map;
  int n, base, v;
  __device__ __forceinline__ void init(const int32_t* m, int n_, int j0, int lane) {
    map = m;
    n = n_;
    base = j0;
    v = map[min(j0 + lane, n - 1)];
  }
  __device__ __forceinline__ int row(int j, int lane) {
    if (j - base >= 64) {
      base = j;
      v = map[min(j + lane, n - 1)];
    }
    return __builtin_amdgcn_readlane(v, j - base) * TK;
  }
};

// floor(n / d) for 0 <= n < 2^24, d >= 1, with inv_d = 1.0f / d: a float
// estimate that is off by at most one, then corrected with integer checks.
__device__ __forceinline__ int div_small(int n, int d, float inv_d) {
  int q = int(float(n) * inv_d);
  q -= q * d > n ? 1 : 0;
  q += (q + 1) * d <= n ? 1 : 0;
  return q;
}

// ------------------------------------------------------------ tile staging
// Tiles are copied from global memory straight into LDS (global_load_lds,
// 16 bytes per lane: lane l of the wave writes LDS bytes [base + 16 l, +16)).
// The copy is issued from inline assembly so that the compiler neither holds
// registers for it nor waits for it before unrelated LDS reads; callers wait
// with lds_dma_wait() before the barrier that publishes the tile. M0 (the LDS
// base of the copy) is saved and restored around it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base));
}

__device__ __forceinline__ void lds_dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's copies are still outstanding (copies
// complete in issue order, so the older ones are done).
template <int N>
__device__ __forceinline__ void lds_dma_wait_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Wait for every outstanding vector-memory load, visibly to the compiler.
// Register loads issued before a tile loop would otherwise stay "pending" in
// the compiler's bookkeeping at the loop header, and it would place a full
// vmcnt(0) inside the loop, where that wait also drains the (invisible)
// prefetch copies of the next tile.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Copy plan of one lane for staging R rows x D elements of a token-major
// tensor into a swizzled LDS tile with NW waves: the lane's 16-byte chunks
// and their element offsets within the source rows, computed once. Rows past
// nrows - 1 repeat row nrows - 1 (callers mask them).
template <typename T, int R, int D, int NW>
struct TileCopy {
  static constexpr int EPC = 16 / int(sizeof(T));
  static constexpr int NCH = D / EPC;
  static constexpr int NT = 64 * NW;
  static constexpr int NC = R * NCH;              // chunks in the tile
  static constexpr int CPW = (NC + NT - 1) / NT;  // copies per lane (the last may be partial)
  static_assert(NC % 64 == 0, "whole waves per copy");
  uint32_t off[CPW];  // element offset of each copy's chunk: r * stride + c * EPC
  int wave, lane;
  int64_t stride;

  __device__ __forceinline__ void init(int wave_, int lane_, int64_t stride_) {
    wave = wave_;
    lane = lane_;
    stride = stride_;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int pos = min(u * NT + wave * 64 + lane, NC - 1);
      const int r = pos / NCH, c = (pos % NCH) ^ tile_swz<NCH>(r);
      off[u] = uint32_t(r * stride + c * EPC);
    }
  }
  // copy u of this wave exists (whole waves: NC is a multiple of 64)
  __device__ __forceinline__ bool has(int u) const {
    if constexpr (NC % NT == 0) return true;
    return u * NT + wave * 64 < NC;
  }
  __device__ __forceinline__ void issue(T* tile, const T* src, int row0, int nrows) const {
    const uint32_t base = lds_addr(tile) + uint32_t(wave * 64) * 16u;
    if (row0 + R <= nrows) {
      const T* s0 = src + (int64_t)row0 * stride;
#pragma unroll
      for (int u = 0; u < CPW; ++u)
        if (has(u)) lds_dma16(s0 + off[u], __builtin_amdgcn_readfirstlane(base + uint32_t(u * NT) * 16u));
    } else {
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        if (!has(u)) continue;
        const int pos = u * NT + wave * 64 + lane;
        const int r = pos / NCH, c = (pos % NCH) ^ tile_swz<NCH>(r);
        const int row = min(row0 + r, nrows - 1);
        lds_dma16(src + (int64_t)row * stride + c * EPC,
                  __builtin_amdgcn_readfirstlane(base + uint32_t(u * NT) * 16u));
      }
    }
  }
};

// Eight floats as two bf16 fragments, x ~ hi + lo: hi = x rounded to bf16,
// lo = the remainder x - hi rounded to bf16 (together about 16 bits of x).
__device__ __forceinline__ void split_pack(const float* x, Elem<true>::Frag& hi,
                                           Elem<true>::Frag& lo) {
  hi = Elem<true>::pack(x);
  const uint32_t h[4] = {hi.v.x, hi.v.y, hi.v.z, hi.v.w};
  float r[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = x[2 * j] - __uint_as_float(h[j] << 16);
    r[2 * j + 1] = x[2 * j + 1] - __uint_as_float(h[j] & 0xffff0000u);
  }
  lo = Elem<true>::pack(r);
}

// Four consecutive output values at element offset `off` of `out`: in the
// element type of E, or as float32 when OF32 (float32 outputs for bf16
// inputs; 16-byte aligned since off is a multiple of 4).
template <class E, bool OF32>
__device__ __forceinline__ void store_out(void* out, int64_t off, float a, float b, float c, float d) {
  if constexpr (OF32) *(float4*)((float*)out + off) = make_float4(a, b, c, d);
  else E::store4((typename E::T*)out + off, a, b, c, d);
}

// Operand reads kept in flight ahead of the matrix product that consumes them.
constexpr int kReadAhead = 3;

// A chain of N matrix products in which product k takes one operand fragment
// read from LDS by read(k) and is issued by mma(k, fragment). The reads run
// PF products ahead of the products, and scheduling fences keep that order.
// Left to itself, the compiler sinks each read next to its product when
// registers are scarce, and every product then waits for a full LDS round
// trip.
// The same chain with hook(k) run right after product k, inside the fenced
// slot: vector work placed there overlaps the products that follow it (a
// wave issues independent vector instructions while its matrix products
// run), instead of waiting for the whole chain.
template <int N, int PF, class Frag, class Read, class Mma, class Hook>
__device__ __forceinline__ void product_chain_hooked(Read read, Mma mma, Hook hook) {
  Frag buf[PF];
#pragma unroll
  for (int k = 0; k < PF && k < N; ++k) buf[k] = read(k);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    mma(k, buf[k % PF]);
    if (k + PF < N) buf[k % PF] = read(k + PF);
    hook(k);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// max of x over lanes l and l ^ 32 (v_permlane32_swap: a register exchange
// between the wave's halves, no LDS round trip)
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int N, int PF, class Frag, class Read, class Mma>
__device__ __forceinline__ void product_chain(Read read, Mma mma) {
  Frag buf[PF];
#pragma unroll
  for (int k = 0; k < PF && k < N; ++k) buf[k] = read(k);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    mma(k, buf[k % PF]);
    if (k + PF < N) buf[k % PF] = read(k + PF);
  }
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace dev
}  // namespace bdattn
