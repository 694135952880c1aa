// Host-side sizing of the mask workspace (plain C++: the ABI layer calls it before any HIP call).
#include <stddef.h>

#include "launch.hpp"
#include "stage_layout.hpp"

namespace sattn {

constexpr size_t SCORE_STAGE_BUDGET = 2048ull << 20;  // bytes of fp32 scores staged per pass

int mask_heads_per_pass(int BH, int G, int Nk) {
  const size_t per = (size_t)G * (size_t)score_stride(Nk) * 4;
  size_t hp = per ? SCORE_STAGE_BUDGET / per : 1;
  if (hp < 1) hp = 1;
  if (hp > (size_t)BH) hp = (size_t)BH;
  return (int)hp;
}

size_t mask_workspace_bytes(int BH, int G, int Nk, int D) {
  const size_t means = align256((size_t)BH * G * D * 2);
  const size_t hp = (size_t)mask_heads_per_pass(BH, G, Nk);
  const size_t scores = align256(hp * G * score_stride(Nk) * 4);
  const size_t samples = align256(hp * G * sample_stride(Nk) * 4);
  return 2 * means + scores + samples;
}

}  // namespace sattn
