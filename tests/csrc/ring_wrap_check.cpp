// CPU build of the ring-head reduction the kernels use (common.h): for every
// stored head v and ring size R it must give the non-negative remainder, a
// slot in [0, R), equal to v for v already in [0, R).  Prints "ok" or the
// first failing case.
#include <stdio.h>

#include "common.h"

int main() {
  for (int R = 1; R <= 7; ++R) {
    for (long long v = -3000; v <= 3000; ++v) {
      const int r = pbsa::ring_wrap((int)v, R);
      const long long want = ((v % R) + R) % R;
      if (r != want || r < 0 || r >= R || (v >= 0 && v < R && r != v)) {
        printf("fail R=%d v=%lld got %d want %lld\n", R, v, r, want);
        return 1;
      }
    }
    const int extremes[] = {INT32_MIN, INT32_MIN + 1, -1, INT32_MAX - 1, INT32_MAX};
    for (int v : extremes) {
      const int r = pbsa::ring_wrap(v, R);
      const long long want = (((long long)v % R) + R) % R;
      if (r != want) {
        printf("fail R=%d v=%d got %d want %lld\n", R, v, r, want);
        return 1;
      }
    }
  }
  printf("ok\n");
  return 0;
}
