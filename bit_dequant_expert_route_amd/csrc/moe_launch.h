// moe_launch.h -- host-side launch-shape helpers shared by the kernel files.
#pragma once

#include <stdio.h>
#include <stdlib.h>

namespace moe_impl {

// ---------------------------------------------------------------------------
// launch shapes
// ---------------------------------------------------------------------------

// Passes per wave (rows per wave = passes * rows per pass) of each kernel.
// MOE_TUNE="gu=<p>,dn=<p>,sh=<p>" (p = 1, 2 or 4) overrides the defaults.
struct Tune {
  int gu = 0, dn = 0, sh = 0;
};
inline const Tune &tune() {
  static const Tune t = [] {
    Tune r;
    const char *e = getenv("MOE_TUNE");
    if (!e) return r;
    for (const char *s = e; *s;) {
      int v = 0;
      if (sscanf(s, "gu=%d", &v) == 1) r.gu = v;
      else if (sscanf(s, "dn=%d", &v) == 1) r.dn = v;
      else if (sscanf(s, "sh=%d", &v) == 1) r.sh = v;
      while (*s && *s != ',') ++s;
      if (*s == ',') ++s;
    }
    return r;
  }();
  return t;
}
inline int pick_pass(int tuned, int dflt) {
  return (tuned == 1 || tuned == 2 || tuned == 4) ? tuned : dflt;
}

// instantiated (NCH, NPASS) pairs: NCH 2 with at most two passes, NCH 4
// (rows wider than 2048 codes per 64 lanes) with one
#define MOE_DISPATCH(nch, npass, ...)                                                    \
  do {                                                                                   \
    if (nch == 1 && npass == 1) { constexpr int NCH_ = 1, NP_ = 1; __VA_ARGS__; }        \
    else if (nch == 1 && npass == 2) { constexpr int NCH_ = 1, NP_ = 2; __VA_ARGS__; }   \
    else if (nch == 1) { constexpr int NCH_ = 1, NP_ = 4; __VA_ARGS__; }                 \
    else if (nch == 2 && npass == 1) { constexpr int NCH_ = 2, NP_ = 1; __VA_ARGS__; }   \
    else if (nch == 2) { constexpr int NCH_ = 2, NP_ = 2; __VA_ARGS__; }                 \
    else { constexpr int NCH_ = 4, NP_ = 1; __VA_ARGS__; }                              \
  } while (0)

}  // namespace moe_impl
