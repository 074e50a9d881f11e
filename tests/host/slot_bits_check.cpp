// Host check of the select kernel's per-lane slot bit sets (slot_bits.h):
// for 1, 64, 65 and 128 slots, every slot set alone reads back alone, in the
// word and bit it belongs to, and a mixed pattern reads back exactly.
#include <cstdio>
#include <vector>

#include "slot_bits.h"

template <int SPL>
int check() {
  int bad = 0;
  for (int e = 0; e < SPL; ++e) {
    bsa::SlotBits<SPL> b;
    b.clear();
    b.set(e);
    for (int f = 0; f < SPL; ++f)
      if (b.get(f) != (f == e)) ++bad;
    for (int q = 0; q < b.NWD; ++q) {
      const unsigned long long want = q == e / 64 ? 1ull << (e % 64) : 0ull;
      if (b.w[q] != want) ++bad;
    }
  }
  bsa::SlotBits<SPL> b;
  b.clear();
  std::vector<bool> ref(SPL, false);
  for (int e = 0; e < SPL; ++e)
    if ((e * 7 + 3) % 5 < 2 || e == SPL - 1 || e == 63 || e == 64) {
      if (e < SPL) {
        b.set(e);
        ref[e] = true;
      }
    }
  for (int e = 0; e < SPL; ++e)
    if (b.get(e) != ref[e]) ++bad;
  std::printf("SPL=%d words=%d mismatches=%d\n", SPL, b.NWD, bad);
  return bad;
}

int main() {
  const int bad = check<1>() + check<64>() + check<65>() + check<128>();
  return bad == 0 ? 0 : 1;
}
