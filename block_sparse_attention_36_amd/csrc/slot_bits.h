// One bit per register slot of a lane for the register form of the select
// kernel (slot e of lane l holds block 64e + l), in as many 64-bit words as SPL
// slots need: slot e is bit e % 64 of word e / 64, so no shift reaches 64.
// Plain constexpr members: the same header compiles for the device (where the
// words live in registers) and for a host check of the indexing.
#pragma once

namespace bsa {

template <int SPL>
struct SlotBits {
  static_assert(SPL >= 1, "at least one slot");
  static constexpr int NWD = (SPL + 63) / 64;
  unsigned long long w[NWD];
  constexpr void clear() {
    for (int q = 0; q < NWD; ++q) w[q] = 0ull;
  }
  constexpr bool get(int e) const { return (w[e >> 6] >> (e & 63)) & 1ull; }
  constexpr void set(int e) { w[e >> 6] |= 1ull << (e & 63); }
};

}  // namespace bsa
