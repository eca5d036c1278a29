/* Test driver: runs the C oracle (oracle/recurrence.c) on inputs read from
 * a file, every array in an allocation of its exact size, so that a build
 * with -fsanitize=address,undefined reports any access outside them.  Used
 * by tests/test_oracle_sanitize.py; not part of the oracle or the library.
 *
 * Input file (native-endian): int64 header[10] = {mode (0 delta rule,
 * 1 decay-only), gate_per_channel, n_seqs, h_qk, h_v, dk, dv, T, has_h0,
 * threads}, int64 cu_seqlens[n_seqs + 1], then float64 q [T h_qk dk],
 * k [T h_qk dk], v [T h_v dv], beta [T h_v] (delta rule only),
 * g [T h_v (dk if per channel)], h0 [n_seqs h_v dk dv] (if has_h0).
 * Output file: float64 o [T h_v dv], then ht [n_seqs h_v dk dv]. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_delta_rule_f64(int kda, int n_seqs, const int64_t* cu_seqlens, int h_qk, int h_v,
                          int dk, int dv, const double* q, const double* k, const double* v,
                          const double* beta, const double* g, const double* h0, double* o,
                          double* ht, int n_threads);
int oracle_decay_f64(int per_channel, int n_seqs, const int64_t* cu_seqlens, int h_qk, int h_v,
                     int dk, int dv, const double* q, const double* k, const double* v,
                     const double* g, const double* h0, double* o, double* ht);

static void* read_block(FILE* f, size_t elems, size_t size) {
  void* p = malloc(elems ? elems * size : 1);
  if (!p || fread(p, size, elems, f) != elems) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s input output\n", argv[0]);
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int64_t* hd = (int64_t*)read_block(f, 10, sizeof(int64_t));
  const int mode = (int)hd[0], pc = (int)hd[1], n = (int)hd[2], h_qk = (int)hd[3],
            h_v = (int)hd[4], dk = (int)hd[5], dv = (int)hd[6], has_h0 = (int)hd[8],
            threads = (int)hd[9];
  const size_t T = (size_t)hd[7];
  int64_t* cu = (int64_t*)read_block(f, (size_t)n + 1, sizeof(int64_t));
  double* q = (double*)read_block(f, T * h_qk * dk, sizeof(double));
  double* k = (double*)read_block(f, T * h_qk * dk, sizeof(double));
  double* v = (double*)read_block(f, T * h_v * dv, sizeof(double));
  double* beta = mode == 0 ? (double*)read_block(f, T * h_v, sizeof(double)) : NULL;
  double* g = (double*)read_block(f, T * h_v * (pc ? dk : 1), sizeof(double));
  double* h0 = has_h0 ? (double*)read_block(f, (size_t)n * h_v * dk * dv, sizeof(double)) : NULL;
  fclose(f);
  const size_t no = T * h_v * dv, nh = (size_t)n * h_v * dk * dv;
  double* o = (double*)malloc(no ? no * sizeof(double) : 1);
  double* ht = (double*)malloc(nh ? nh * sizeof(double) : 1);
  int rc = mode == 0
               ? oracle_delta_rule_f64(pc, n, cu, h_qk, h_v, dk, dv, q, k, v, beta, g, h0, o, ht,
                                       threads)
               : oracle_decay_f64(pc, n, cu, h_qk, h_v, dk, dv, q, k, v, g, h0, o, ht);
  if (rc != 0) {
    fprintf(stderr, "oracle rejected the arguments\n");
    return 3;
  }
  FILE* out = fopen(argv[2], "wb");
  if (!out || fwrite(o, sizeof(double), no, out) != no || fwrite(ht, sizeof(double), nh, out) != nh)
    return 2;
  fclose(out);
  free(hd); free(cu); free(q); free(k); free(v); free(beta); free(g); free(h0); free(o); free(ht);
  return 0;
}
