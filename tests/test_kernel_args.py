"""The host and the kernels agree on the step arguments, read from the
sources: the kernels' parameter list (MK_STEP_PARAMS), the array of
argument addresses the host launch passes (kernel_launch's params[]), the
aggregate that rebuilds the argument struct inside a kernel (MK_STEP_ARGS)
and the struct itself (Args) name the same fields in the same order with the
same types.  A mismatch would hand a kernel one argument in another's place,
which nothing on the host would notice."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "persistent_interpreter_amd", "csrc")


def _strip_comments(s):
    s = re.sub(r"/\*.*?\*/", "", s, flags=re.S)
    return re.sub(r"//[^\n]*", "", s)


def _norm_type(t):
    t = re.sub(r"\b(const|__restrict__)\b", "", t)
    return re.sub(r"\s+", "", t)


def _args_struct():
    src = _strip_comments(open(os.path.join(CSRC, "mk_plan.hpp")).read())
    body = re.search(r"struct Args\s*\{(.*?)\};", src, flags=re.S).group(1)
    fields = []
    for decl in body.split(";"):
        decl = " ".join(decl.split())
        if not decl:
            continue
        m = re.match(r"(.*?[\s*])(\w+(?:\s*,\s*\w+)*)$", decl)
        base = m.group(1)
        for name in m.group(2).split(","):
            fields.append((name.strip(), _norm_type(base)))
    return fields


def _kernel_src():
    return _strip_comments(open(os.path.join(CSRC, "mk_kernel.hip")).read())


def _macro(src, name):
    m = re.search(r"#define " + name + r"(\([^)]*\))?\s*((?:[^\n]*\\\n)*[^\n]*)", src)
    return m.group(2).replace("\\\n", " ")


def test_kernel_parameters_follow_the_argument_struct():
    fields = _args_struct()
    assert fields[-1][0] == "step_off"          # set inside the kernel only
    params = []
    for p in _macro(_kernel_src(), "MK_STEP_PARAMS").split(","):
        m = re.match(r"\s*(.*?[\s*])(\w+)\s*$", p)
        params.append((m.group(2), _norm_type(m.group(1))))
    assert params == fields[:-1]


def test_launch_passes_every_field_in_order():
    src = _kernel_src()
    body = re.search(r"void \*params\[\]\s*=\s*\{(.*?)\};", src, flags=re.S).group(1)
    names = [re.match(r"\s*&a\.(\w+)\s*$", x).group(1) for x in body.split(",")]
    assert names == [f for f, _ in _args_struct()[:-1]]


def test_kernel_rebuilds_the_struct_in_field_order():
    agg = _macro(_kernel_src(), "MK_STEP_ARGS")
    inside = re.search(r"Args\s*\{(.*)\}", agg).group(1)
    names = [x.strip() for x in inside.split(",")]
    expect = [f for f, _ in _args_struct()]
    expect[expect.index("n_steps")] = "NS"        # the launch's step count
    expect[expect.index("step_off")] = "0"
    assert names == expect
