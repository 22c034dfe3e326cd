"""Readers for the hand-derived golden fixtures in this folder (plain text)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _lines(name):
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def masks():
    """{(workload, step): [[...], ...]}"""
    out, cur, rows = {}, None, []
    for line in _lines("masks.txt"):
        if line.startswith("mask "):
            _, name, _, step = line.split()
            cur, rows = (name, int(step)), []
        elif line == "end":
            out[cur] = rows
            cur = None
        else:
            rows.append([int(x) for x in line.split()])
    return out


def fresh_columns():
    out = {}
    for line in _lines("fresh_columns.txt"):
        head, cols = line.split(":")
        name, step, row = head.split()
        out[(name, int(step), int(row))] = [int(x) for x in cols.split()]
    return out


def counts():
    out = {}
    for line in _lines("counts.txt"):
        head, vals = line.split(":")
        name, step = head.split()
        out[(name, int(step))] = [int(x) for x in vals.split()]
    return out
