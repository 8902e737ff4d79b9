/* planted_overflow.c -- reads one element past a heap array on purpose.  The
 * host-sanitizer test loads it to show that the sanitizer run really reports
 * such a read (CPU only; nothing here touches a GPU). */
#include <stdlib.h>

int planted_read_past_end(int n) {
  volatile int *a = malloc(sizeof(int) * (size_t)n);
  for (int i = 0; i < n; ++i) a[i] = i;
  int v = a[n];  /* one past the end */
  free((void *)a);
  return v;
}
