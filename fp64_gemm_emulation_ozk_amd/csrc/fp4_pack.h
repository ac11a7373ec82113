// Shared pieces of the FP4 plane packers.
//
// Every FP4 engine stores an integer operand as a few planes of e2m1 codes (4 bits each),
// two codes per byte with the lower K index in the low nibble, so that a 16-byte fragment
// holds 32 consecutive K values of one plane.  A packer looks every value up in a table of
// its plane codes and writes the planes out.  The table here holds one 32-bit "spread"
// word per value: byte t carries the code of plane t in its low nibble (planes 0..3).  Two
// neighbouring values then make the byte of every plane at once (word | next << 4), and
// four such pair words give the 32-bit words of the four planes by a 4 x 4 byte transpose
// (eight v_perm_b32), about 4 vector instructions per value in all.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ozk {

// Byte t of the result = nibble t of c (t = 0..3).
__host__ __device__ constexpr uint32_t spread_nibbles(uint32_t c) {
  return (c & 0xFu) | ((c & 0xF0u) << 4) | ((c & 0xF00u) << 8) | ((c & 0xF000u) << 12);
}

// Spread words of 8 consecutive values -> the first NP (<= 4) plane words: nibble u of
// word t is plane t's code of value u.
template <int NP>
__device__ __forceinline__ void pack8_planes(const uint32_t (&s)[8], uint32_t (&w)[NP]) {
  static_assert(NP >= 1 && NP <= 4, "at most 4 planes per spread word");
  uint32_t p[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) p[k] = s[2 * k] | (s[2 * k + 1] << 4);   // byte t: plane t's pair
  // rows p0..p3 of a 4 x 4 byte matrix; plane t's word is its column t
  const uint32_t x0 = __builtin_amdgcn_perm(p[1], p[0], 0x05010400u);  // p0.0 p1.0 p0.1 p1.1
  const uint32_t y0 = __builtin_amdgcn_perm(p[3], p[2], 0x05010400u);  // p2.0 p3.0 p2.1 p3.1
  w[0] = __builtin_amdgcn_perm(y0, x0, 0x05040100u);
  if constexpr (NP > 1) w[1] = __builtin_amdgcn_perm(y0, x0, 0x07060302u);
  if constexpr (NP > 2) {
    const uint32_t x1 = __builtin_amdgcn_perm(p[1], p[0], 0x07030602u);  // p0.2 p1.2 p0.3 p1.3
    const uint32_t y1 = __builtin_amdgcn_perm(p[3], p[2], 0x07030602u);
    w[2] = __builtin_amdgcn_perm(y1, x1, 0x05040100u);
    if constexpr (NP > 3) w[3] = __builtin_amdgcn_perm(y1, x1, 0x07060302u);
  }
}

// Byte c (0..3) of the dword w, masked to the table size (mask 255 for int8 values indexed
// by their unsigned byte, 15 for int4 values by their low nibble).
__device__ __forceinline__ uint32_t byte_of(uint32_t w, int c, uint32_t mask) {
  return (w >> (8 * c)) & mask;
}

// Coalesced store of one item of NP 16-byte pieces per lane (a line's K step) through this
// wave's LDS area: `stage` holds 64 items of 16 NP bytes, `dsts` 64 destinations.  Lane i
// puts its pieces (piece p in slot (p + i) mod NP, so that the lanes of one write spread
// over the banks) and its destination (nullptr: nothing to store) there; then store
// instruction j writes pieces 64 j .. 64 j + 63 of the 64 NP in item order, 16
// consecutive bytes per lane, so every instruction covers whole items instead of 16 bytes
// of 64 of them.  All 64 lanes must call it.
template <int NP>
__device__ __forceinline__ void wave_staged_store(uint4* stage, uint8_t** dsts,
                                                  const uint4 (&piece)[NP], uint8_t* dst) {
  const int lane = threadIdx.x & 63;
  const int rot = lane % NP;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int slot = p + rot < NP ? p + rot : p + rot - NP;
    stage[lane * NP + slot] = piece[p];
  }
  dsts[lane] = dst;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int q = 64 * j + lane;
    const int item = q / NP, p = q - item * NP;
    const int r = item % NP;
    const int slot = p + r < NP ? p + r : p + r - NP;
    uint8_t* d = dsts[item];
    const uint4 v = stage[item * NP + slot];
    if (d) *reinterpret_cast<uint4*>(d + 16 * p) = v;
  }
  // the area is free for the next call once every lane has read it
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace ozk
