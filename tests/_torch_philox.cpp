// Test helper: exposes PyTorch's own Philox4x32-10 engine (ATen's
// PhiloxRNGEngine.h, an implementation independent of the oracle's) through a
// C symbol, so the oracle's dropout stream can be pinned against it.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>

extern "C" void torch_philox4(uint64_t seed, uint64_t subsequence, uint64_t offset, uint32_t* out) {
  // Key = seed; counter words 0-1 = offset, words 2-3 = subsequence.
  at::Philox4_32 eng(seed, subsequence, offset);
  for (int i = 0; i < 4; ++i) out[i] = eng();
}
