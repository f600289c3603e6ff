/* CPython fast-call entry points for the reduction calls (and the launch-floor hooks) of
 * libargreduce.so.
 *
 * Argument marshalling only, like the ctypes binding it sits beside: each function takes
 * the C ABI's arguments as Python ints (device pointers, enum codes, sizes, the stream
 * handle), converts them, and calls the library through a function pointer that the
 * binding hands over from its loaded copy of the library (bind()), so this module links
 * against nothing but the Python runtime. The point is the cost per call: a ctypes call
 * with nine converted arguments takes about 2 us of host time, which is as long as the
 * GPU needs for a small reduction; a METH_FASTCALL function takes a small fraction of it.
 *
 * The reduction calls release the GIL while the library enqueues (as ctypes does), so host
 * threads can launch side by side.
 *
 * Return value: the library's status code as a Python int. A Python argument that is not
 * an int in range raises TypeError / OverflowError before the library is called; calling
 * before bind() raises RuntimeError.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include "argreduce.h"

typedef int (*lastaxis_fn)(const void *, argreduce_dtype_t, int64_t, int64_t, argreduce_op_t,
                           int64_t *, void *, size_t, void *);
typedef int (*axis_fn)(const void *, argreduce_dtype_t, int64_t, int64_t, int64_t,
                       argreduce_op_t, int64_t *, void *, size_t, void *);
typedef int (*scan_fn)(const void *, argreduce_dtype_t, int64_t, int64_t, argreduce_op_t,
                       void *, int64_t *, void *, size_t, void *);

typedef int (*empty_fn)(void *);
typedef int (*store_fn)(int64_t *, void *);
typedef int (*read_fn)(const void *, size_t, uint32_t *, int64_t, void *);

static lastaxis_fn g_lastaxis = NULL;
static axis_fn g_axis = NULL;
static scan_fn g_scan = NULL;
static empty_fn g_empty = NULL;
static store_fn g_store = NULL;
static read_fn g_read = NULL;

/* An address from a Python int (0 for NULL). */
static void *arg_ptr(PyObject *o) { return PyLong_AsVoidPtr(o); }

static int check_bound(const void *fn) {
    if (fn == NULL) {
        PyErr_SetString(PyExc_RuntimeError, "argreduce fast calls used before bind()");
        return -1;
    }
    return 0;
}

static int check_nargs(Py_ssize_t got, Py_ssize_t want, const char *name) {
    if (got != want) {
        PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, want, got);
        return -1;
    }
    return 0;
}

/* argreduce_lastaxis(x, dtype, rows, cols, op, out_idx, scratch, scratch_bytes, stream) */
static PyObject *fast_lastaxis(PyObject *self, PyObject *const *a, Py_ssize_t n) {
    (void)self;
    if (check_nargs(n, 9, "argreduce_lastaxis") || check_bound((const void *)g_lastaxis))
        return NULL;
    const void *x = arg_ptr(a[0]);
    const long dtype = PyLong_AsLong(a[1]);
    const long long rows = PyLong_AsLongLong(a[2]);
    const long long cols = PyLong_AsLongLong(a[3]);
    const long op = PyLong_AsLong(a[4]);
    int64_t *out = (int64_t *)arg_ptr(a[5]);
    void *scratch = arg_ptr(a[6]);
    const size_t sbytes = PyLong_AsSize_t(a[7]);
    void *stream = arg_ptr(a[8]);
    if (PyErr_Occurred()) return NULL;
    int rc;
    Py_BEGIN_ALLOW_THREADS
    rc = g_lastaxis(x, (argreduce_dtype_t)dtype, (int64_t)rows, (int64_t)cols,
                    (argreduce_op_t)op, out, scratch, sbytes, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(rc);
}

/* argreduce_axis(x, dtype, outer, len, inner, op, out_idx, scratch, scratch_bytes, stream) */
static PyObject *fast_axis(PyObject *self, PyObject *const *a, Py_ssize_t n) {
    (void)self;
    if (check_nargs(n, 10, "argreduce_axis") || check_bound((const void *)g_axis)) return NULL;
    const void *x = arg_ptr(a[0]);
    const long dtype = PyLong_AsLong(a[1]);
    const long long outer = PyLong_AsLongLong(a[2]);
    const long long len = PyLong_AsLongLong(a[3]);
    const long long inner = PyLong_AsLongLong(a[4]);
    const long op = PyLong_AsLong(a[5]);
    int64_t *out = (int64_t *)arg_ptr(a[6]);
    void *scratch = arg_ptr(a[7]);
    const size_t sbytes = PyLong_AsSize_t(a[8]);
    void *stream = arg_ptr(a[9]);
    if (PyErr_Occurred()) return NULL;
    int rc;
    Py_BEGIN_ALLOW_THREADS
    rc = g_axis(x, (argreduce_dtype_t)dtype, (int64_t)outer, (int64_t)len, (int64_t)inner,
                (argreduce_op_t)op, out, scratch, sbytes, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(rc);
}

/* argreduce_scan_lastaxis(x, dtype, rows, cols, op, out_values, out_idx, scratch,
 *                         scratch_bytes, stream) */
static PyObject *fast_scan(PyObject *self, PyObject *const *a, Py_ssize_t n) {
    (void)self;
    if (check_nargs(n, 10, "argreduce_scan_lastaxis") || check_bound((const void *)g_scan))
        return NULL;
    const void *x = arg_ptr(a[0]);
    const long dtype = PyLong_AsLong(a[1]);
    const long long rows = PyLong_AsLongLong(a[2]);
    const long long cols = PyLong_AsLongLong(a[3]);
    const long op = PyLong_AsLong(a[4]);
    void *values = arg_ptr(a[5]);
    int64_t *out = (int64_t *)arg_ptr(a[6]);
    void *scratch = arg_ptr(a[7]);
    const size_t sbytes = PyLong_AsSize_t(a[8]);
    void *stream = arg_ptr(a[9]);
    if (PyErr_Occurred()) return NULL;
    int rc;
    Py_BEGIN_ALLOW_THREADS
    rc = g_scan(x, (argreduce_dtype_t)dtype, (int64_t)rows, (int64_t)cols, (argreduce_op_t)op,
                values, out, scratch, sbytes, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(rc);
}

/* The measurement hooks, marshalled the same way so that their floors carry the same
 * host cost per call as the reductions they are compared with. */

/* argreduce_debug_launch_empty(stream) */
static PyObject *fast_empty(PyObject *self, PyObject *const *a, Py_ssize_t n) {
    (void)self;
    if (check_nargs(n, 1, "argreduce_debug_launch_empty") || check_bound((const void *)g_empty))
        return NULL;
    void *stream = arg_ptr(a[0]);
    if (PyErr_Occurred()) return NULL;
    return PyLong_FromLong(g_empty(stream));
}

/* argreduce_debug_launch_store(out, stream) */
static PyObject *fast_store(PyObject *self, PyObject *const *a, Py_ssize_t n) {
    (void)self;
    if (check_nargs(n, 2, "argreduce_debug_launch_store") || check_bound((const void *)g_store))
        return NULL;
    int64_t *out = (int64_t *)arg_ptr(a[0]);
    void *stream = arg_ptr(a[1]);
    if (PyErr_Occurred()) return NULL;
    return PyLong_FromLong(g_store(out, stream));
}

/* argreduce_debug_launch_read(x, bytes, out, grid, stream) */
static PyObject *fast_read(PyObject *self, PyObject *const *a, Py_ssize_t n) {
    (void)self;
    if (check_nargs(n, 5, "argreduce_debug_launch_read") || check_bound((const void *)g_read))
        return NULL;
    const void *x = arg_ptr(a[0]);
    const size_t bytes = PyLong_AsSize_t(a[1]);
    uint32_t *out = (uint32_t *)arg_ptr(a[2]);
    const long long grid = PyLong_AsLongLong(a[3]);
    void *stream = arg_ptr(a[4]);
    if (PyErr_Occurred()) return NULL;
    return PyLong_FromLong(g_read(x, bytes, out, (int64_t)grid, stream));
}

/* bind(lastaxis, axis, scan_lastaxis, debug_launch_empty, debug_launch_store,
 *      debug_launch_read): the library's entry points, as addresses. */
static PyObject *fast_bind(PyObject *self, PyObject *const *a, Py_ssize_t n) {
    (void)self;
    if (check_nargs(n, 6, "bind")) return NULL;
    void *p[6];
    for (int k = 0; k < 6; ++k) p[k] = arg_ptr(a[k]);
    if (PyErr_Occurred()) return NULL;
    for (int k = 0; k < 6; ++k) {
        if (p[k] == NULL) {
            PyErr_SetString(PyExc_ValueError, "bind() needs six non-null addresses");
            return NULL;
        }
    }
    g_lastaxis = (lastaxis_fn)p[0];
    g_axis = (axis_fn)p[1];
    g_scan = (scan_fn)p[2];
    g_empty = (empty_fn)p[3];
    g_store = (store_fn)p[4];
    g_read = (read_fn)p[5];
    Py_RETURN_NONE;
}

static PyMethodDef k_methods[] = {
    {"bind", (PyCFunction)(void (*)(void))fast_bind, METH_FASTCALL,
     "bind(lastaxis, axis, scan_lastaxis, debug_launch_empty, debug_launch_store, "
     "debug_launch_read): the library entry points to call, as addresses."},
    {"argreduce_debug_launch_empty", (PyCFunction)(void (*)(void))fast_empty, METH_FASTCALL,
     "argreduce_debug_launch_empty(stream)"},
    {"argreduce_debug_launch_store", (PyCFunction)(void (*)(void))fast_store, METH_FASTCALL,
     "argreduce_debug_launch_store(out, stream)"},
    {"argreduce_debug_launch_read", (PyCFunction)(void (*)(void))fast_read, METH_FASTCALL,
     "argreduce_debug_launch_read(x, bytes, out, grid, stream)"},
    {"argreduce_lastaxis", (PyCFunction)(void (*)(void))fast_lastaxis, METH_FASTCALL,
     "argreduce_lastaxis(x, dtype, rows, cols, op, out_idx, scratch, scratch_bytes, stream)"},
    {"argreduce_axis", (PyCFunction)(void (*)(void))fast_axis, METH_FASTCALL,
     "argreduce_axis(x, dtype, outer, len, inner, op, out_idx, scratch, scratch_bytes, "
     "stream)"},
    {"argreduce_scan_lastaxis", (PyCFunction)(void (*)(void))fast_scan, METH_FASTCALL,
     "argreduce_scan_lastaxis(x, dtype, rows, cols, op, out_values, out_idx, scratch, "
     "scratch_bytes, stream)"},
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef k_module = {PyModuleDef_HEAD_INIT, "_argreduce_fast",
                                      "Fast-call marshalling for libargreduce.so.", -1,
                                      k_methods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__argreduce_fast(void) { return PyModule_Create(&k_module); }
