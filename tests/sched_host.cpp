// Host-only build of the launch-schedule arithmetic in csrc/sched.hpp (the
// same header the kernels and launchers use), exported with C linkage for
// the schedule tests.  Compiled by the tests with the host C++ compiler.
#include "sched.hpp"

using namespace gptq::sched;

extern "C" {

int64_t chol_rest_tiles(int k, int T) { return rest_tiles(k, T); }

void chol_rest_tile(int k, int64_t b, int64_t* i, int64_t* j) { rest_tile(k, b, *i, *j); }

int chol_paired_default(int T) { return chol_paired(T) ? 1 : 0; }

void chol_launch_geom(int k, int T, int paired, int64_t* out) {
    const CholLaunch g = chol_launch(k, T, paired != 0);
    out[0] = g.nchain;
    out[1] = g.n_rest;
    out[2] = g.grid;
}

int far_split_c(int64_t n_units, int n_sweep, int n_cu, int64_t c_begin, int nstrip, int64_t* out) {
    FarSplit fs;
    fs.c_begin = c_begin;
    fs.nstrip = nstrip;
    const int nf = far_split(n_units, n_sweep, n_cu, fs);
    out[0] = fs.n_units;
    out[1] = fs.per_sweep;
    out[2] = fs.q;
    out[3] = fs.r;
    return nf;
}

void far_units_c(int64_t n_units, int n_sweep, int n_cu, int64_t c_begin, int nstrip, int b, int64_t* u0,
                 int64_t* u1) {
    FarSplit fs;
    fs.c_begin = c_begin;
    fs.nstrip = nstrip;
    far_split(n_units, n_sweep, n_cu, fs);
    far_units(fs, b, n_sweep, *u0, *u1);
}

void far_sub_c(int64_t n_units, int n_sweep, int n_cu, int64_t c_begin, int nstrip, int64_t u, int64_t u1,
               int64_t d_in, int64_t* out) {
    FarSplit fs;
    fs.c_begin = c_begin;
    fs.nstrip = nstrip;
    far_split(n_units, n_sweep, n_cu, fs);
    const FarSub t = far_sub(fs, u, u1, d_in);
    out[0] = t.rt;
    out[1] = t.c0;
    out[2] = t.c_end;
    out[3] = t.ns;
}

int far_constants(int* rows, int* cols, int* strip) {
    *rows = kFarRows;
    *cols = kFarCols;
    *strip = kFarStrip;
    return 0;
}

}  // extern "C"
