// LDS staging primitives shared by the libpab attention kernels (gfx950):
// XOR-swizzled tile rows, LDS-DMA copy plans (buffer_load ... lds) and the
// waits and barriers that keep such copies in flight.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pab {

typedef __attribute__((address_space(3))) void lds_void_t;

// Slot of 16-byte chunk c of row r in a swizzled LDS tile with CPR chunks per
// row is c ^ swz(r).  Every operand read below has the 16 lanes of one LDS
// phase read the same chunk index of 16 consecutive rows; the swizzle sends
// them to 16 disjoint 4-bank groups.
template <int CPR>
__device__ constexpr int swz(int row) {
  return CPR == 16 ? (row & 15) : CPR == 8 ? ((row >> 1) & 7) : CPR == 4 ? ((row >> 2) & 3)
                                                                          : ((row >> 3) & 1);
}

// Lane offsets of the LDS-DMA copy of a region of rows (16 CPR bytes each,
// gstride bytes apart in HBM).  Instruction `inst` fills region bytes
// [1024 inst, 1024 inst + 1024), lane i writing 16 bytes at 1024 inst + 16 i
// and fetching the global chunk that belongs in that slot.  The swizzle of
// row inst * RPI + lane / CPR depends on inst only through inst % PER.
template <int CPR>
struct DmaPlan {
  static constexpr int RPI = 64 / CPR;                            // rows per instruction
  static constexpr int PER = CPR == 16 ? 4 : CPR == 8 ? 2 : 1;    // swizzle period
  uint32_t off[PER];
  __device__ void init(int lane, int64_t gstride) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int row = p * RPI + lane / CPR;
      off[p] = (uint32_t)((lane / CPR) * gstride + 16 * ((lane % CPR) ^ swz<CPR>(row)));
    }
  }
};

#if defined(__HIP_DEVICE_COMPILE__)
constexpr int kRsrcWord3 = 0x00020000;   // raw byte buffer

// Workgroup barrier that does not wait for outstanding LDS-DMA copies (a
// plain __syncthreads() fences every memory operation, including the copies
// that are meant to stay in flight); this wave's LDS reads are complete first.
// The waits use the s_waitcnt builtin (simm16: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8) rather than inline asm so that the compiler's own
// wait-count tracking sees them and adds no conservative waits of its own.
__device__ inline void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Waits until at most N of this wave's LDS-DMA copies are outstanding.
template <int N>
__device__ inline void wait_vm_le() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

#endif  // __HIP_DEVICE_COMPILE__

}  // namespace pab
