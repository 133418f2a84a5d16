// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// vector types, the matrix-core (MFMA) operations used, the LDS transpose
// read, and small numeric helpers.
//
// Matrix-core lane layouts (wave64), as used throughout:
//
//  v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//    A: lane l holds row (l % 32), k = 8*(l / 32) + 0..7     (8 x bf16)
//    B: lane l holds col (l % 32), k = 8*(l / 32) + 0..7     (8 x bf16)
//    C: lane l, element i holds row 8*(i/4) + 4*(l/32) + (i%4), col (l % 32)
//
//  v_mfma_f32_32x32x2_f32    C[32x32] += A[32x2] * B[2x32]
//    A: lane l holds row (l % 32), k = l / 32;  B: col (l % 32), k = l / 32
//    C: as above.
//
//  v_mfma_f32_16x16x4_f32    C[16x16] += A[16x4] * B[4x16]
//    A: lane l holds row (l % 16), k = l / 16;  B: col (l % 16), k = l / 16
//    C: lane l, element i holds row 4*(l/16) + i, col (l % 16)
//
//  ds_read_b64_tr_b16: within each group of 16 lanes, lane 4r+j supplies the
//    address of 4 consecutive 16-bit values = row r, columns 4j..4j+3 of a
//    4 x 16 tile; lane i of the group receives column i (rows 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32_16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// `p` must point into LDS (a __shared__ array); it is converted to the LDS
// address space for the instruction.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS bf16x4*)(const_cast<__bf16*>(p)));
}

// The same reads at an LDS byte address held as an integer (a per-lane base
// plus a constant the compiler folds into the instruction's 16-bit offset).
__device__ __forceinline__ bf16x8 lds_load16_at(uint32_t addr) {
  return *reinterpret_cast<const FA_LDS bf16x8*>((uintptr_t)addr);
}
__device__ __forceinline__ bf16x4 lds_read_tr16_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<FA_LDS bf16x4*>((uintptr_t)addr));
}

// Direct global -> LDS copy of 16 bytes per lane: lane j's 16 bytes at
// base + voffset land at LDS byte address lds_addr + 16 j.  Issued from
// inline assembly so that the compiler does not treat the copy as an LDS
// store aliasing every later LDS read (it would wait for the copy before the
// first one); the caller therefore waits for the copies itself
// (s_waitcnt vmcnt(0)) before they are read.  The instruction has no result
// registers, and M0 is set and used inside the same block.
#pragma clang diagnostic push
// M0 is reserved; nothing else in these kernels keeps a value in it across
// the copy (LDS reads and lane shuffles do not use M0 on gfx950).
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(uint32_t lds_addr, const void* base, uint32_t voffset) {
  // Both scalar operands are wave-uniform; the read-first-lane makes that
  // visible to the compiler where its divergence analysis cannot prove it.
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  base = (const void*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                                  (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_addr), "v"(voffset), "s"(base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(0): every vector-memory load of this wave has completed,
// the LDS copies above included.  Written with the builtin so that the
// compiler's own wait tracking knows that its earlier loads are done too.
__device__ __forceinline__ void wait_lds_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): all but the last N vector-memory loads of this wave
// have completed (they complete in issue order), e.g. one block's copies
// done while the next block's N are still in flight.
template <int N>
__device__ __forceinline__ void wait_lds_dma_but() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that leaves vector-memory loads (the LDS copies above)
// in flight.  It waits only for this wave's own LDS reads (lgkmcnt(0)), so
// that a buffer read before the barrier may be refilled after it; the asm
// statement's memory clobber keeps the compiler from moving memory accesses
// across it and the scheduling barriers keep every instruction on its side.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Fixes the point where x is computed: the compiler may not sink its
// computation past this statement (towards a later use) nor hoist it above
// an earlier one.  Emits no instruction.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

// Accumulators of fp32 matrix products (AGPR form) made safe to read after
// the loop that built them.  On a loop-exit path the compiler's wait-state
// count for "matrix product writes a register, vector instruction reads it"
// has been seen to fall short (the epilogue read the last accumulator
// register 7 wait states after the final 16-pass product, and got the value
// from before it).  Here 32 wait states pass inside a statement that takes
// every accumulator in its AGPRs, so any later read (the copy to VGPRs
// included) depends on the wait.
// Every accumulator is an operand of the one statement that holds the
// wait, so no product that writes one can be scheduled after the wait.
template <int N>
__device__ __forceinline__ void settle_acc(f32x16 (&acc)[N]) {
  static_assert(N == 1 || N == 2 || N == 4, "one, two or four accumulators");
  if constexpr (N == 1) {
    asm volatile("s_nop 15\n\ts_nop 15" : "+a"(acc[0]));
  } else if constexpr (N == 2) {
    asm volatile("s_nop 15\n\ts_nop 15" : "+a"(acc[0]), "+a"(acc[1]));
  } else {
    asm volatile("s_nop 15\n\ts_nop 15"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
  }
}
// Same for two accumulator sets built in the same loop.
template <int N>
__device__ __forceinline__ void settle_acc(f32x16 (&x)[N], f32x16 (&y)[N]) {
  static_assert(N == 1 || N == 2 || N == 4, "one, two or four accumulators");
  if constexpr (N == 1) {
    asm volatile("s_nop 15\n\ts_nop 15" : "+a"(x[0]), "+a"(y[0]));
  } else if constexpr (N == 2) {
    asm volatile("s_nop 15\n\ts_nop 15" : "+a"(x[0]), "+a"(x[1]), "+a"(y[0]), "+a"(y[1]));
  } else {
    asm volatile("s_nop 15\n\ts_nop 15"
                 : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]),
                   "+a"(y[0]), "+a"(y[1]), "+a"(y[2]), "+a"(y[3]));
  }
}

// ---- bf16 products with the register file of each operand chosen here
// In a kernel that needs more than the 256 vector registers, the compiler
// gives every product the accumulation registers (AGPRs) for its result, and
// vector code that reads a result copies it back one register at a time.
// Written as inline assembly, a product whose result the vector code reads
// (scores) can keep it in vector registers, with its constant B operand in
// AGPRs.  The compiler counts no wait states around inline assembly: a
// kernel using these fences each product's result (fence_results) before
// any read of it; the vector writes of their A operands are loads, which the
// compiler's own s_waitcnt covers.  The hazard check on the built assembly
// verifies every path.

// c = a b (zero accumulator): c in vector registers, b in AGPRs.
__device__ __forceinline__ f32x16 mfma_bf16_v0(bf16x8 a, bf16x8 b) {
  f32x16 c;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
  return c;
}
// c += a b: c in vector registers, b in AGPRs.
__device__ __forceinline__ void mfma_bf16_v(f32x16& c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
// 12 wait states inside a statement that takes the two results x and y, so
// every later read of them depends on it; placed after the last product that
// writes them.
__device__ __forceinline__ void fence_results(f32x16& x, f32x16& y) {
  asm volatile("s_nop 11" : "+v"(x), "+v"(y));
}

// An index given either as a compile-time constant (std::integral_constant)
// or as a run-time int.
template <typename X>
__device__ __forceinline__ constexpr int value_of(X x) {
  if constexpr (std::is_integral_v<X>) return x;
  else return X::value;
}

// Calls f(std::integral_constant<int, I>{}) for I = BEGIN .. END-1, so that
// the index is a compile-time constant in the body.
template <int BEGIN, int END, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (BEGIN < END) {
    f(std::integral_constant<int, BEGIN>{});
    static_for<BEGIN + 1, END>(f);
  }
}

template <typename T>
__device__ __forceinline__ uint32_t lds_address(const T* p) {
  return (uint32_t)(uintptr_t)((FA_LDS const void*)p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// The two halves of the wave combined, the result in every lane: lane l and
// lane l ^ 32 both get op(x[l mod 32], x[l mod 32 + 32]).  v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; with x as both operands one result holds x's lower half twice and
// the other x's upper half twice.  A register-to-register move, unlike a
// shuffle through the LDS unit, so it does not wait behind LDS reads.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  lo = __builtin_bit_cast(float, (uint32_t)r[0]);
  hi = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

// Round-to-nearest-even float -> bf16 pair.
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return r;
}

// Two floats rounded to bf16 (RNE) in one 32-bit register, a in the low half:
// one v_cvt_pk_bf16_f32.  Four such words form an 8 x bf16 operand.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, to_bf16x2(a, b));
}
__device__ __forceinline__ bf16x8 bf16x8_of(const u32x4& w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

template <typename T, typename U>
__device__ __forceinline__ T bit_cast(const U& u) {
  static_assert(sizeof(T) == sizeof(U), "size mismatch");
  return __builtin_bit_cast(T, u);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// Map a linear workgroup id to a work index so that consecutive work indices
// land on the same XCD (workgroups are dispatched round-robin over the XCDs).
// Work indices [x*per, (x+1)*per) run on XCD x.  Falls back to the identity
// when the grid does not split evenly.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  if (total % kXcds != 0) return bid;
  const int per = total / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

// Work order for tiles of unequal cost (under the causal mask the query
// tiles near the end and the key tiles near the start see the most keys or
// queries): block `bid` of `total` = heads * n_tiles gets (head, rank), rank 0
// being a head's costliest tile.  Blocks go round-robin over the XCDs; each
// XCD gets whole heads (their K/V stay in one L2) and issues its tiles
// costliest first across all of its heads, so that no large tile starts
// last while the other compute units idle.  Without an even split of the
// heads over the XCDs the order is costliest first over all heads.
__device__ __forceinline__ void costliest_first(int bid, int total, int n_tiles, int& head, int& rank) {
  const int heads = total / n_tiles;
  if (heads % kXcds == 0) {
    const int per = heads / kXcds;
    const int i = bid / kXcds;
    head = (bid % kXcds) * per + i % per;
    rank = i / per;
  } else {
    head = bid % heads;
    rank = bid / heads;
  }
}

}  // namespace fa
