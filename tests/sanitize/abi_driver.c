/*
 * Host-side driver of the C ABI for the sanitizer builds: reads one call per
 * line from stdin, "<exported name> <integer arguments...> <expected
 * result>" (the stream argument is left out and passed as NULL), makes the
 * call (every one of them returns before any device work: argument
 * checks, size queries, status strings) and prints each mismatch and a
 * count.
 * Pointer arguments are passed as integers (fake, never dereferenced
 * addresses; 0 is NULL).  Exit status: the number of mismatches.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mxgemm.h"

#define PTR(x) ((void *)(uintptr_t)(x))

int main(void) {
  char line[4096];
  int bad = 0, n = 0;
  while (fgets(line, sizeof line, stdin)) {
    char name[64];
    long long a[24];
    int off = 0, k = 0;
    if (sscanf(line, "%63s%n", name, &off) != 1) continue;
    char *p = line + off;
    while (k < 24) {
      char *end;
      long long v = strtoll(p, &end, 0);
      if (end == p) break;
      a[k++] = v;
      p = end;
    }
    if (k < 1) { printf("malformed: %s", line); ++bad; continue; }   /* at least the expected result */
    const long long expect = a[k - 1];
    const int na = k - 1;
    long long got = 0;
    if (!strcmp(name, "mxgemm_validate") && na == 11) {
      got = mxgemm_validate((int)a[0], (int)a[1], (int)a[2], PTR(a[3]), PTR(a[4]), PTR(a[5]), PTR(a[6]),
                            PTR(a[7]), a[8], a[9], a[10]);
    } else if (!strcmp(name, "mxgemm_run") && na == 11) {
      got = mxgemm_run((int)a[0], (int)a[1], (int)a[2], PTR(a[3]), PTR(a[4]), PTR(a[5]), PTR(a[6]),
                       PTR(a[7]), a[8], a[9], a[10], NULL);
    } else if (!strcmp(name, "mxgemm_validate_fused") && na == 13) {
      got = mxgemm_validate_fused((int)a[0], (int)a[1], (int)a[2], PTR(a[3]), PTR(a[4]), PTR(a[5]),
                                  PTR(a[6]), PTR(a[7]), a[8], a[9], a[10], PTR(a[11]), (int)a[12]);
    } else if (!strcmp(name, "mxgemm_run_fused") && na == 13) {
      got = mxgemm_run_fused((int)a[0], (int)a[1], (int)a[2], PTR(a[3]), PTR(a[4]), PTR(a[5]), PTR(a[6]),
                             PTR(a[7]), a[8], a[9], a[10], PTR(a[11]), (int)a[12], NULL);
    } else if (!strcmp(name, "grouped_fp8_gemm_validate") && na == 11) {
      got = grouped_fp8_gemm_validate((int)a[0], (const int64_t *)PTR(a[1]), PTR(a[2]), PTR(a[3]),
                                      PTR(a[4]), PTR(a[5]), PTR(a[6]), a[7], a[8], a[9], (int)a[10]);
    } else if (!strcmp(name, "grouped_fp8_gemm_run") && na == 11) {
      got = grouped_fp8_gemm_run((int)a[0], (const int64_t *)PTR(a[1]), PTR(a[2]), PTR(a[3]), PTR(a[4]),
                                 PTR(a[5]), PTR(a[6]), a[7], a[8], a[9], (int)a[10], NULL);
    } else if (!strcmp(name, "grouped_fp8_gemm_autotune") && na == 14) {
      got = grouped_fp8_gemm_autotune((int)a[0], (const int64_t *)PTR(a[1]), PTR(a[2]), PTR(a[3]), PTR(a[4]),
                                      PTR(a[5]), PTR(a[6]), a[7], a[8], a[9], (int)a[10], (int)a[11],
                                      (int *)PTR(a[12]), (float *)PTR(a[13]), NULL);
    } else if (!strcmp(name, "mxgemm_tune_cache_size") && na == 0) {
      got = mxgemm_tune_cache_size();
    } else if (!strcmp(name, "mxgemm_preshuffle_b_bytes") && na == 3) {
      got = mxgemm_preshuffle_b_bytes((int)a[0], a[1], a[2]);
    } else if (!strcmp(name, "mxgemm_preshuffle_scales_bytes") && na == 2) {
      got = mxgemm_preshuffle_scales_bytes(a[0], a[1]);
    } else if (!strcmp(name, "mxgemm_preshuffle_b") && na == 6) {
      got = mxgemm_preshuffle_b((int)a[0], (int)a[1], PTR(a[2]), PTR(a[3]), a[4], a[5], NULL);
    } else if (!strcmp(name, "mxgemm_preshuffle_scales") && na == 4) {
      got = mxgemm_preshuffle_scales(PTR(a[0]), PTR(a[1]), a[2], a[3], NULL);
    } else if (!strcmp(name, "grouped_bf16_gemm_validate") && na == 9) {
      got = grouped_bf16_gemm_validate((int)a[0], (const int64_t *)PTR(a[1]), PTR(a[2]), PTR(a[3]),
                                       PTR(a[4]), a[5], a[6], a[7], (int)a[8]);
    } else if (!strcmp(name, "grouped_bf16_gemm_run") && na == 9) {
      got = grouped_bf16_gemm_run((int)a[0], (const int64_t *)PTR(a[1]), PTR(a[2]), PTR(a[3]), PTR(a[4]),
                                  a[5], a[6], a[7], (int)a[8], NULL);
    } else if (!strcmp(name, "grouped_bf16_preshuffle_b") && na == 5) {
      got = grouped_bf16_preshuffle_b((int)a[0], PTR(a[1]), PTR(a[2]), a[3], a[4], NULL);
    } else if (!strcmp(name, "grouped_fp8_preshuffle_b") && na == 5) {
      got = grouped_fp8_preshuffle_b((int)a[0], PTR(a[1]), PTR(a[2]), a[3], a[4], NULL);
    } else if (!strcmp(name, "mxgemm_quantize_mx") && na == 6) {
      got = mxgemm_quantize_mx((int)a[0], (const float *)PTR(a[1]), PTR(a[2]), PTR(a[3]), a[4], a[5], NULL);
    } else if (!strcmp(name, "mxgemm_quantize_tensor") && na == 5) {
      got = mxgemm_quantize_tensor((int)a[0], (const float *)PTR(a[1]), PTR(a[2]), (float *)PTR(a[3]), a[4],
                                   NULL);
    } else if (!strcmp(name, "grouped_fp8_quantize_act") && na == 7) {
      got = grouped_fp8_quantize_act((int)a[0], (const int64_t *)PTR(a[1]), (const float *)PTR(a[2]),
                                     PTR(a[3]), (float *)PTR(a[4]), a[5], a[6], NULL);
    } else if (!strcmp(name, "grouped_fp8_quantize_weight") && na == 6) {
      got = grouped_fp8_quantize_weight((int)a[0], (const float *)PTR(a[1]), PTR(a[2]), (float *)PTR(a[3]),
                                        a[4], a[5], NULL);
    } else if (!strcmp(name, "mxgemm_status_string") && na == 1) {
      const char *s = mxgemm_status_string((int)a[0]);
      got = (s != NULL && strlen(s) > 0) ? expect : -999;
    } else {
      printf("unknown call or argument count: %s", line);
      ++bad;
      continue;
    }
    ++n;
    if (got != expect) {
      printf("MISMATCH %s -> %lld, expected %lld\n", name, got, expect);
      ++bad;
    }
  }
  printf("%d calls, %d mismatches\n", n, bad);
  return bad > 255 ? 255 : bad;
}
